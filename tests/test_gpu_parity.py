"""GPU parity of the HIP path against the float64 oracle.

The library is called through the C ABI (ctypes binding).  Bars: max rel err
(max_i |x_i - y_i| / max_i |y_i| per tensor) <= 1e-4 in fp32 I/O mode and
<= 2e-2 in bf16 mode, on O and on the final W1, W2, W3 (and M), after all
chunks.  Full-size workloads run every pair on the GPU and compare sampled
(batch, head) pairs with the oracle (pairs are independent).
"""

import numpy as np
import pytest

import lact_synth as S
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

TINY = S.WORKLOADS["tiny"]


def small(base, **kw):
    kw.setdefault("name", f"{base}-small")
    return S.WORKLOADS[base].replace(**kw)


SMALL_CASES = [
    TINY,
    TINY.replace(name="tiny-uta", order="update_then_apply"),
    TINY.replace(name="tiny-momentum", opt="momentum", beta=0.9),
    TINY.replace(name="tiny-muon", opt="muon"),
    TINY.replace(name="tiny-muon-momentum", opt="muon", beta=0.5, order="update_then_apply"),
    # ragged chunks: 3 chunks of 300 keys (not a multiple of any tile), 50 queries
    TINY.replace(name="tiny-ragged", T_kv=900, chunk_kv=300, T_q=150, chunk_q=50, opt="muon"),
    TINY.replace(name="fp32-d128", B=2, H=2, d=128, h=256, opt="momentum", beta=0.9),
    TINY.replace(name="fp32-d32", B=1, H=3, d=32, h=64, opt="muon"),
    TINY.replace(name="fp32-d64-h256", H=2, h=256, opt="gd", order="update_then_apply"),
    small("lm", B=2, H=2, T_kv=4096, T_q=4096, chunk_kv=1024, chunk_q=1024),
    small("posed", H=2, T_kv=16384, T_q=512, chunk_kv=16384, chunk_q=512),
    small("video", H=2, T_kv=3 * 4096, T_q=3 * 4096),
    small("million", H=2, T_kv=40000, T_q=1000, chunk_kv=40000, chunk_q=1000),
    # bf16, chunks shorter than one LDS stage of the MFMA kernel, ragged
    small("posed", name="posed-tiny-chunks", H=3, T_kv=1000, T_q=70, chunk_kv=100, chunk_q=7,
          opt="momentum", beta=0.9),
    # the same under Muon: on 100-key chunks Newton-Schulz lifts the weak
    # directions of the gradient, where bf16 operand rounding alone moves the
    # result by ~7e-2, so the default product precision (auto) keeps the derived
    # operands split here
    small("posed", name="posed-tiny-chunks-muon", H=3, T_kv=300, T_q=21, chunk_kv=100,
          chunk_q=7, products="auto"),
    # the video workload's shape and length under the default product precision
    # (14 Muon chunks: split products)
    small("video", name="video-auto", H=1, products="auto"),
    # bf16, two 128-unit hidden slices at d = 64; 1000 queries (two query-read
    # workgroups of several pipelined 128-query steps, the last one ragged)
    small("posed", name="posed-h256", H=2, h=256, T_kv=5000, T_q=1000, chunk_kv=5000, chunk_q=1000),
    # split products at d = 64 (one wavefront per SIMD): one posed-shape chunk, a
    # ragged eight-chunk Muon scan (auto keeps the products split over more than four
    # Muon chunks) and a rate per token and matrix
    small("posed", name="posed-split", H=2, T_kv=16384, T_q=512, chunk_kv=16384, chunk_q=512,
          products="split"),
    small("posed", name="posed-split-scan", H=2, T_kv=8000, T_q=400, chunk_kv=1000, chunk_q=50,
          products="auto"),
    small("posed", name="posed-split-eta3", H=2, T_kv=3000, T_q=210, chunk_kv=1000, chunk_q=70,
          opt="momentum", beta=0.9, eta_per_matrix=True, products="split"),
    # bf16 Muon with momentum at d = 64 (the Muon tail's momentum buffer)
    small("posed", name="posed-muon-momentum", H=2, T_kv=9000, T_q=256, chunk_kv=9000, chunk_q=256,
          beta=0.5),
    # split products at d = 128, chunks of 1000 keys (ragged against the 64-token stage)
    small("video", name="video-ragged", H=2, T_kv=3000, T_q=3000, chunk_kv=1000, chunk_q=1000),
    # split products with momentum under Muon
    small("video", name="video-muon-momentum", H=1, T_kv=2 * 4096, T_q=2 * 4096, beta=0.5),
    # bf16 at d = 128 with four 128-unit hidden slices, ragged chunks
    small("lm", name="lm-h512-ragged", B=1, H=2, h=512, T_kv=3000, T_q=600, chunk_kv=1500,
          chunk_q=300),
    # d = 128 with bf16 products on the two-wavefront kernel (128-unit hidden slices): three
    # slices (h = 384) with ragged chunks, and one (h = 128)
    small("lm", name="lm-h384-ragged", B=1, H=2, h=384, T_kv=3000, T_q=600, chunk_kv=1500,
          chunk_q=300),
    small("lm", name="lm-h128", B=2, H=1, h=128, T_kv=2048, T_q=512, chunk_kv=1024, chunk_q=256),
    # chunks shorter than one LDS stage of the d = 128 kernel (64 keys with bf16 products,
    # 32 with split products; Muon over ten 20-key chunks takes split products)
    small("lm", name="lm-tiny-chunks", B=1, H=2, T_kv=300, T_q=60, chunk_kv=30, chunk_q=6),
    small("video", name="video-tiny-chunks", H=2, T_kv=200, T_q=40, chunk_kv=20, chunk_q=4,
          products="auto"),
    # rows kept at their length (norm_mode LACT_NORM_KEEP) through every update tail:
    # fp32 GD / momentum (row-wise tail), fp32 Muon (step-and-normalise kernel), bf16
    # momentum (16-byte row-group tail), bf16 Muon at d = 64 and split-product Muon at
    # d = 128 (Newton-Schulz tails)
    TINY.replace(name="tiny-keep", norm="keep"),
    TINY.replace(name="tiny-muon-keep", opt="muon", norm="keep", order="update_then_apply"),
    TINY.replace(name="fp32-d128-keep", B=1, H=2, d=128, h=256, opt="momentum", beta=0.9,
                 norm="keep"),
    small("lm", name="lm-keep", B=1, H=2, T_kv=4096, T_q=4096, chunk_kv=1024, chunk_q=1024,
          norm="keep"),
    small("posed", name="posed-keep", H=2, T_kv=16384, T_q=512, chunk_kv=16384, chunk_q=512,
          norm="keep"),
    small("video", name="video-keep", H=1, T_kv=2 * 4096, T_q=2 * 4096, norm="keep"),
    # a learning rate per token and matrix (eta_mode LACT_ETA_PER_MATRIX), in every gradient
    # kernel: fp32 generic (d = 64 and 128), bf16 MFMA at d = 64, bf16 and split-product MFMA
    # at d = 128; ragged chunks for the stage logic
    TINY.replace(name="tiny-eta3", eta_per_matrix=True, opt="momentum", beta=0.9),
    TINY.replace(name="fp32-d128-eta3", B=1, H=2, d=128, h=256, opt="muon", eta_per_matrix=True),
    small("posed", name="posed-eta3", H=2, T_kv=16384, T_q=512, chunk_kv=16384, chunk_q=512,
          eta_per_matrix=True),
    small("posed", name="posed-eta3-ragged", H=3, T_kv=3000, T_q=210, chunk_kv=1000, chunk_q=70,
          opt="momentum", beta=0.9, eta_per_matrix=True),
    small("lm", name="lm-eta3", B=1, H=2, T_kv=3000, T_q=3000, chunk_kv=1500, chunk_q=1500,
          eta_per_matrix=True),
    small("video", name="video-eta3", H=1, T_kv=2 * 4096, T_q=2 * 4096, eta_per_matrix=True),
]


@pytest.mark.parametrize("w", SMALL_CASES, ids=[w.name for w in SMALL_CASES])
def test_small_parity(w):
    G.say(f"case {w.name}")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O, st_gpu = G.run_gpu(w, x, st)
    O_ref, st_ref = G.run_oracle(w, x, st)
    _, bad = G.compare(w, O, st_gpu, O_ref, st_ref)
    assert not bad, bad


def random_case(seed):
    """A seeded draw over the supported shapes and options (sizes small enough for
    the oracle): head dim, hidden width, I/O type, optimizer, order, ragged chunk
    sizes and the two variants, with the default product precision (auto)."""
    r = np.random.default_rng(1000 + seed)
    d = int(r.choice([32, 64, 128]))
    h = int(r.choice([32, 64, 96, 128, 160, 256, 384]))
    io = str(r.choice(["fp32", "bf16"]))
    opt = str(r.choice(["gd", "momentum", "muon"]))
    n_chunks = int(r.integers(1, 4))
    chunk_kv = int(r.integers(40, 1600))
    chunk_q = int(r.integers(1, 300))
    return TINY.replace(
        name=f"random-{seed}", B=int(r.integers(1, 3)), H=int(r.integers(1, 3)), d=d, h=h,
        io_dtype=io, opt=opt, beta=float(r.choice([0.0, 0.5, 0.9])) if opt != "gd" else 0.0,
        order=str(r.choice(["apply_then_update", "update_then_apply"])),
        T_kv=n_chunks * chunk_kv, chunk_kv=chunk_kv, T_q=n_chunks * chunk_q, chunk_q=chunk_q,
        norm=str(r.choice(["unit", "keep"])), eta_per_matrix=bool(r.integers(0, 2)), seed=seed)


@pytest.mark.parametrize("seed", range(12))
def test_random_config_parity(seed):
    w = random_case(seed)
    G.say(f"case {w}")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O, st_gpu = G.run_gpu(w, x, st)
    O_ref, st_ref = G.run_oracle(w, x, st)
    _, bad = G.compare(w, O, st_gpu, O_ref, st_ref)
    assert not bad, bad


FULL = [
    ("posed", [(0, 0), (0, 4), (0, 7), (0, 11)], {}),
    ("million", [(0, 3), (0, 10)], {}),
    ("lm", [(0, 0), (2, 5), (5, 3), (7, 7)], {}),
    ("video", [(0, 0), (0, 13), (0, 26), (0, 39)], {}),
    # split products at d = 64 (the route of long or short-chunk Muon scans) at full size
    ("posed", [(0, 2), (0, 9)], {"products": "split"}),
    ("million", [(0, 6)], {"products": "split"}),
    # the variants at full size
    ("posed", [(0, 5)], {"eta_per_matrix": True}),
    ("lm", [(2, 6)], {"norm": "keep"}),
]


@pytest.mark.parametrize("name,pairs,variant", FULL,
                         ids=[f[0] + "".join(f"-{k}" for k in f[2]) for f in FULL])
def test_full_size_sampled_parity(name, pairs, variant):
    w = S.WORKLOADS[name].replace(**variant)
    G.say(f"case {name} full size, oracle pairs {pairs}")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O, st_gpu = G.run_gpu(w, x, st)
    O_ref, st_ref = G.run_oracle(w, x, st, pairs=pairs)
    _, bad = G.compare(w, O, st_gpu, O_ref, st_ref, pairs=pairs)
    assert not bad, bad
    # properties that hold for every pair: unit rows (or the initial lengths), finite outputs
    for n in ("W1", "W2", "W3"):
        norms = np.linalg.norm(st_gpu[n], axis=-1)
        want = np.linalg.norm(st[n], axis=-1) if w.norm == "keep" else 1.0
        assert np.max(np.abs(norms - want)) < 1e-4, n
    assert np.all(np.isfinite(O))


def test_deterministic_repeat():
    w = SMALL_CASES[10]
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O1, s1 = G.run_gpu(w, x, st)
    O2, s2 = G.run_gpu(w, x, st)
    assert np.array_equal(O1, O2)
    for n in s1:
        assert np.array_equal(s1[n], s2[n]), n


def test_resume_split_run_is_bitwise_equal():
    import torch
    import chunk_test_amd as L
    w = small("lm", B=1, H=2, T_kv=4096, T_q=4096, chunk_kv=1024, chunk_q=1024)
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O_full, s_full = G.run_gpu(w, x, st)
    cfg = G.config_of(w)
    dst = G.device_state(w, st)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = G.to_dev(x["eta"], w, io=False)
    ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
    O = torch.empty_like(Q)
    for lo, hi in ((0, 2048), (2048, 4096)):
        q, k, v = (t[:, :, lo:hi].contiguous() for t in (Q, K, V))
        e = eta[:, :, lo:hi].contiguous()
        o = torch.empty_like(q)
        L.lact_chunked_forward(cfg, dst, q, k, v, e, o, w.chunk_kv, w.chunk_q, w.order, ws)
        O[:, :, lo:hi] = o
    torch.cuda.synchronize()
    assert np.array_equal(O.float().cpu().numpy(), O_full)
    for n in s_full:
        assert np.array_equal(dst[n].cpu().numpy(), s_full[n]), n


def test_scan_weight_copy_matches_per_chunk_calls():
    """Inside the chunk scan each query read loads the bf16 weight copy that
    the update tail (here the Muon tail) wrote; per-chunk lact_update +
    lact_apply calls convert the fp32 weights instead.  Same bits."""
    import torch
    import chunk_test_amd as L
    w = small("posed", name="copy", H=2, T_kv=2 * 4096, T_q=2 * 256, chunk_kv=4096, chunk_q=256)
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O_scan, s_scan = G.run_gpu(w, x, st)
    cfg = G.config_of(w)
    dst = G.device_state(w, st)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = G.to_dev(x["eta"], w, io=False)
    ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
    O = torch.empty_like(Q)
    for c in range(2):
        kv = slice(c * w.chunk_kv, (c + 1) * w.chunk_kv)
        qs = slice(c * w.chunk_q, (c + 1) * w.chunk_q)
        k, v, e = (t[:, :, kv].contiguous() for t in (K, V, eta))
        q = Q[:, :, qs].contiguous()
        o = torch.empty_like(q)
        L.lact_update(cfg, dst, k, v, e, ws)
        L.lact_apply(cfg, dst, q, o, ws=ws)
        O[:, :, qs] = o
    torch.cuda.synchronize()
    assert np.array_equal(O.float().cpu().numpy(), O_scan)
    for n in ("W1", "W2", "W3"):
        assert np.array_equal(dst[n].cpu().numpy(), s_scan[n]), n


@pytest.mark.parametrize("base,kw", [
    ("video", dict(H=3, T_kv=4 * 1024, T_q=4 * 512, chunk_kv=1024, chunk_q=512)),
    ("posed", dict(B=2, H=5, T_kv=3 * 2048, T_q=3 * 300, chunk_kv=2048, chunk_q=300,
                   order="apply_then_update", beta=0.5)),
    ("lm", dict(B=1, H=4, T_kv=4 * 1024, T_q=4 * 512, chunk_kv=1024, chunk_q=512)),
    ("posed", dict(B=3, H=3, T_kv=3 * 2048, T_q=3 * 200, chunk_kv=2048, chunk_q=200,
                   order="apply_then_update", opt="gd")),
    # one chunk (the shared launch from the first chunk on), and 3P = 198 tail
    # workgroups (above the 192 that leave room for the read: separate launches)
    ("posed", dict(H=2, T_kv=2048, T_q=17, chunk_kv=2048, chunk_q=17, order="apply_then_update")),
    ("posed", dict(B=6, H=11, T_kv=2 * 1024, T_q=2 * 64, chunk_kv=1024, chunk_q=64,
                   order="apply_then_update")),
], ids=["muon-d128-h256", "muon-momentum-d64-h128-ragged", "momentum-d128-h256", "gd-d64-h128-ragged",
        "muon-one-chunk", "muon-66-pairs"])
def test_scan_fused_read_matches_per_chunk_calls(base, kw):
    """Apply-then-update scans whose query reads load the bf16 weight copy the
    previous update tail wrote; with the matrix-core Muon tail, from the
    second chunk on, each chunk's tail and query read run in one launch (the
    read loads the copy of the chunk's weights while the tail writes the next
    ones).  Per-chunk lact_apply + lact_update calls (separate launches, fp32
    weights converted on the fly) give the same bits."""
    import torch
    import chunk_test_amd as L
    w = small(base, name=f"fused-{base}", **kw)
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O_scan, s_scan = G.run_gpu(w, x, st)
    cfg = G.config_of(w)
    dst = G.device_state(w, st)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = G.to_dev(x["eta"], w, io=False)
    ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
    O = torch.empty_like(Q)
    for c in range(w.T_kv // w.chunk_kv):
        kv = slice(c * w.chunk_kv, (c + 1) * w.chunk_kv)
        qs = slice(c * w.chunk_q, (c + 1) * w.chunk_q)
        k, v, e = (t[:, :, kv].contiguous() for t in (K, V, eta))
        q = Q[:, :, qs].contiguous()
        o = torch.empty_like(q)
        L.lact_apply(cfg, dst, q, o, ws=ws)
        L.lact_update(cfg, dst, k, v, e, ws)
        O[:, :, qs] = o
    torch.cuda.synchronize()
    assert np.array_equal(O.float().cpu().numpy(), O_scan)
    for n in s_scan:
        assert np.array_equal(dst[n].cpu().numpy(), s_scan[n]), n


def test_update_and_apply_entry_points_and_strided_views():
    import torch
    import chunk_test_amd as L
    w = TINY.replace(name="entry", H=2, opt="muon")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    cfg = G.config_of(w)
    # one chunk via the scan
    w1 = w.replace(T_kv=256, T_q=256)
    x1 = {k: (v[:, :, :256] if v.ndim >= 3 else v).copy() for k, v in x.items()}
    O_scan, s_scan = G.run_gpu(w1, x1, st)
    # the same chunk through lact_apply + lact_update on strided views of
    # the full-length tensors
    dst = G.device_state(w, st)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = G.to_dev(x["eta"], w, io=False)
    ws = L.alloc_workspace(cfg, 256, 256)
    O = torch.zeros_like(Q)
    L.lact_apply(cfg, dst, Q, O, ws=ws, m=256, q_stride_bh=w.T_q * w.d)
    L.lact_update(cfg, dst, K, V, eta, ws, n=256, kv_stride_bh=w.T_kv * w.d, eta_stride_bh=w.T_kv)
    torch.cuda.synchronize()
    assert np.array_equal(O[:, :, :256].cpu().numpy(), O_scan)
    assert np.all(O[:, :, 256:].cpu().numpy() == 0)  # nothing written past m
    for n in ("W1", "W2", "W3"):
        assert np.array_equal(dst[n].cpu().numpy(), s_scan[n]), n


def test_per_matrix_rates_on_chunk_views_match_the_scan():
    """lact_update on views into one [3, B, H, T] rate tensor (pair stride T,
    the three blocks B*H*T apart) gives the scan's result bit for bit."""
    import torch
    import chunk_test_amd as L
    w = small("posed", name="eta3-views", H=2, T_kv=2 * 4096, T_q=2 * 256, chunk_kv=4096,
              chunk_q=256, eta_per_matrix=True, opt="momentum", beta=0.9,
              order="apply_then_update")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O_scan, s_scan = G.run_gpu(w, x, st)
    cfg = G.config_of(w)
    dst = G.device_state(w, st)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = G.to_dev(x["eta"], w, io=False)  # [3, B, H, T_kv]
    ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
    O = torch.empty_like(Q)
    for c in range(2):
        qs = slice(c * w.chunk_q, (c + 1) * w.chunk_q)
        q = Q[:, :, qs].contiguous()
        o = torch.empty_like(q)
        L.lact_apply(cfg, dst, q, o, ws=ws)
        O[:, :, qs] = o
        # strided views: keys/values and rates of chunk c inside the full tensors
        off = c * w.chunk_kv
        L.lact_update(cfg, dst, K[:, :, off:], V[:, :, off:], eta[..., off:], ws, n=w.chunk_kv,
                      kv_stride_bh=w.T_kv * w.d, eta_stride_bh=w.T_kv)
    torch.cuda.synchronize()
    assert np.array_equal(O.float().cpu().numpy(), O_scan)
    for n in ("W1", "W2", "W3", "M1", "M2", "M3"):
        assert np.array_equal(dst[n].cpu().numpy(), s_scan[n]), n


@pytest.mark.parametrize("opt,norm", [("momentum", "unit"), ("momentum", "keep"),
                                      ("muon", "unit"), ("muon", "keep")])
def test_unaligned_state_parity(opt, norm):
    """Weights and momentum 4 bytes past a 16-byte boundary: the row-wise
    tails with 4-byte accesses (GD / momentum) and the fp32-arithmetic Muon
    path (the MFMA Muon tail needs 16-byte rows) against the oracle."""
    import torch
    import chunk_test_amd as L
    w = small("lm", name=f"unaligned-{opt}-{norm}", B=1, H=2, T_kv=2048, T_q=2048, chunk_kv=1024,
              chunk_q=1024, opt=opt, beta=0.9 if opt == "momentum" else 0.0, norm=norm)
    G.say(f"case {w.name}")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    cfg = G.config_of(w)
    dst = {}
    for n in ("W1", "W2", "W3"):
        buf = torch.zeros(st[n].size + 1, device="cuda")
        dst[n] = buf[1:].view(st[n].shape)
        dst[n].copy_(torch.from_numpy(st[n]))
        assert dst[n].data_ptr() % 16 != 0
    if cfg.uses_momentum():
        for n in ("M1", "M2", "M3"):
            buf = torch.zeros(dst["W" + n[1]].numel() + 1, device="cuda")
            dst[n] = buf[1:].view(dst["W" + n[1]].shape)
    Q, K, V = (G.to_dev(x[n], w) for n in ("Q", "K", "V"))
    eta = G.to_dev(x["eta"], w, io=False)
    O = torch.empty_like(Q)
    ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
    L.lact_chunked_forward(cfg, dst, Q, K, V, eta, O, w.chunk_kv, w.chunk_q, w.order, ws)
    torch.cuda.synchronize()
    s_gpu = {n: t.cpu().numpy() for n, t in dst.items()}
    O_ref, s_ref = G.run_oracle(w, x, st)
    _, bad = G.compare(w, O.float().cpu().numpy(), s_gpu, O_ref, s_ref)
    assert not bad, bad


def test_edge_sizes_one_token_one_query():
    w = TINY.replace(name="one-token", T_kv=3, chunk_kv=1, T_q=3, chunk_q=1, opt="muon")
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O, s = G.run_gpu(w, x, st)
    O_ref, s_ref = G.run_oracle(w, x, st)
    _, bad = G.compare(w, O, s, O_ref, s_ref)
    assert not bad, bad


def test_eta_zero_leaves_normalised_initial_weights():
    w = small("posed", H=2, T_kv=4096, T_q=256, chunk_kv=4096, chunk_q=256)
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    x["eta"][:] = 0.0
    O, s = G.run_gpu(w, x, st)
    for n in ("W1", "W2", "W3"):
        ref = st[n] / np.linalg.norm(st[n].astype(np.float64), axis=-1, keepdims=True)
        assert G.rel_err(s[n], ref) < 1e-6, n


def test_invalid_arguments_raise_without_launching():
    import torch
    import chunk_test_amd as L
    import dataclasses
    w = TINY
    cfg = dataclasses.replace(G.config_of(w), d=60)
    st = {n: torch.zeros((1, 1) + ((60, w.h) if n == "W2" else (w.h, 60)), device="cuda")
          for n in ("W1", "W2", "W3")}
    Q = torch.zeros(1, 1, 8, 60, device="cuda")
    with pytest.raises(L.LactError) as e:
        L.lact_apply(cfg, st, Q, torch.empty_like(Q))
    assert e.value.status == -2


def test_offset_buffers_take_the_fp32_kernels_within_tolerance():
    """The launch plan depends on buffer alignment: K, V, Q, O one element past
    a 16-byte boundary run the fp32-arithmetic kernels instead of the matrix
    cores.  Expected: both runs within the bf16 bar of the oracle (not the
    same bits), and each run reproducible bit for bit."""
    import torch
    import chunk_test_amd as L
    w = small("posed", name="offset", H=2, T_kv=4096, T_q=256, chunk_kv=4096, chunk_q=256)
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    cfg = G.config_of(w)
    O_ref, s_ref = G.run_oracle(w, x, st)
    results = []
    for off in (0, 1, 0, 1):
        dst = G.device_state(w, st)
        dev = {}
        for n in ("Q", "K", "V"):
            a = torch.from_numpy(np.ascontiguousarray(x[n])).to(torch.bfloat16)
            buf = torch.zeros(a.numel() + 8, dtype=torch.bfloat16, device="cuda")
            dev[n] = buf[off:off + a.numel()].view(a.shape)
            dev[n].copy_(a)
        obuf = torch.zeros(dev["Q"].numel() + 8, dtype=torch.bfloat16, device="cuda")
        O = obuf[off:off + dev["Q"].numel()].view(dev["Q"].shape)
        assert (dev["K"].data_ptr() % 16 == 0) == (off == 0)
        eta = G.to_dev(x["eta"], w, io=False)
        ws = L.alloc_workspace(cfg, w.chunk_kv, w.chunk_q)
        L.lact_chunked_forward(cfg, dst, dev["Q"], dev["K"], dev["V"], eta, O, w.chunk_kv,
                               w.chunk_q, w.order, ws)
        torch.cuda.synchronize()
        s_np = {n: t.cpu().numpy() for n, t in dst.items()}
        O_np = O.float().cpu().numpy()
        _, bad = G.compare(w, O_np, s_np, O_ref, s_ref)
        assert not bad, (off, bad)
        results.append((O_np, s_np))
    for a, b in ((0, 2), (1, 3)):
        assert np.array_equal(results[a][0], results[b][0])
        for n in results[a][1]:
            assert np.array_equal(results[a][1][n], results[b][1][n]), n
    assert not np.array_equal(results[0][0], results[1][0])


@pytest.mark.parametrize("where", ["eta", "K"])
def test_nan_input_propagates_within_its_pair(where):
    """A NaN in one token's rate (or key) of one pair: that pair's gradient,
    update and weights become NaN and so does every output read after the
    update; every other pair gives the same bits as without the NaN (pairs are
    independent; nothing checks values on the device)."""
    w = small("posed", name=f"nan-{where}", H=3, T_kv=8192, T_q=256, chunk_kv=4096, chunk_q=128)
    st = S.gen_weights(w)
    x = S.gen_inputs(w)
    O0, s0 = G.run_gpu(w, x, st)
    bad_pair = 1
    if where == "eta":
        x["eta"][0, bad_pair, 777] = np.nan
    else:
        x["K"][0, bad_pair, 777, 5] = np.nan
    O1, s1 = G.run_gpu(w, x, st)
    for n in ("W1", "W2", "W3"):
        assert np.all(np.isnan(s1[n][0, bad_pair])), n
        for p in (0, 2):
            assert np.array_equal(s1[n][0, p], s0[n][0, p]), (n, p)
    # update-then-apply: every query of the pair reads the poisoned weights
    assert np.all(np.isnan(O1[0, bad_pair]))
    for p in (0, 2):
        assert np.array_equal(O1[0, p], O0[0, p]), p
