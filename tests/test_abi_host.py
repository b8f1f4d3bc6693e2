"""Host-side checks of the C ABI (no GPU needed: nothing here launches a kernel).

* the library loads and exports every function include/lact.h declares;
* workspace sizing;
* argument validation returns the documented status before any HIP call;
* the binding checks shapes and devices before calling the library.

Several checks hand the library stand-in device addresses (256) with one bad
argument.  Where no GPU is visible a validation regression then ends as a HIP
error (no device); on a machine with a GPU it would launch kernels on those
addresses, so the module runs only where no GPU is visible.
"""

import ctypes
import os
import re

import pytest

import chunk_test_amd as L
from chunk_test_amd import lact as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0  # counts without initialising the runtime
    except Exception:  # noqa: BLE001
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="stand-in device addresses: CPU-only module")


def header_functions():
    text = open(os.path.join(ROOT, "include", "lact.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lact_\w+)\s*\(", text)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("lact_update", "lact_apply", "lact_chunked_forward", "lact_workspace_bytes",
                 "lact_status_string"):
        assert name in fns


def test_library_exports_every_declared_symbol():
    lib = L.load_library()
    for name in header_functions():
        assert hasattr(lib, name), f"{name} not exported"
    assert set(header_functions()) == set(B.EXPORTED)


def test_version_and_status_strings():
    lib = L.load_library()
    assert lib.lact_version() >= 1
    for rc in (0, -1, -2, -3, -4):
        assert lib.lact_status_string(rc).decode()


def test_config_default_matches_python_defaults():
    lib = L.load_library()
    c = B.LactConfig()
    lib.lact_config_default(ctypes.byref(c))
    py = B.Config(B=0, H=0, d=0, h=0).to_c()
    for f, _ in B.LactConfig._fields_:
        assert abs(getattr(c, f) - getattr(py, f)) <= 1e-6 * max(1.0, abs(getattr(py, f))), f


def test_workspace_bytes():
    small = L.workspace_bytes(L.Config(1, 1, 64, 128, io_dtype="fp32"), 256, 256)
    big = L.workspace_bytes(L.Config(1, 12, 64, 128, opt="muon"), 196608, 4096)
    assert small > 0 and big > small
    assert small % 256 == 0 and big % 256 == 0
    # monotone in the chunk size
    c = L.Config(8, 8, 128, 256, opt="momentum", beta=0.9)
    sizes = [L.workspace_bytes(c, n, n) for n in (1, 100, 2048, 100000)]
    assert sizes == sorted(sizes)


def test_unsupported_shapes_report_unsupported():
    lib = L.load_library()
    for d, h in ((100, 128), (64, 100), (256, 512), (64, 2048)):
        c = L.Config(1, 1, d, h).to_c()
        assert lib.lact_workspace_bytes(ctypes.byref(c), 128, 128) == 0
        assert L.mfma_path(d, h) == -1


def _call_update(cfg, st=None, K=1, V=1, eta=1, n=16, kvs=None, es=None, ws=256, wsb=1 << 30):
    lib = L.load_library()
    c = cfg.to_c()
    s = st if st is not None else B.LactState(256, 256, 256, 256, 256, 256)
    kvs = n * cfg.d if kvs is None else kvs
    es = n if es is None else es
    return lib.lact_update(ctypes.byref(c), ctypes.byref(s), K, V, eta, n, kvs, es, ws, wsb, None)


def test_update_validation():
    ok = L.Config(1, 1, 64, 128, io_dtype="fp32")
    lib = L.load_library()
    assert _call_update(L.Config(0, 1, 64, 128)) == B.LACT_ERR_INVALID_ARG
    assert _call_update(L.Config(1, 1, 64, 128, opt="momentum", beta=1.0)) == B.LACT_ERR_INVALID_ARG
    assert _call_update(L.Config(1, 1, 64, 128, opt="momentum", beta=-0.1)) == B.LACT_ERR_INVALID_ARG
    assert _call_update(L.Config(1, 1, 64, 128, norm_eps=0.0)) == B.LACT_ERR_INVALID_ARG
    assert _call_update(L.Config(1, 1, 64, 128, opt="muon", ns_iters=40)) == B.LACT_ERR_INVALID_ARG
    assert _call_update(L.Config(1, 1, 60, 128)) == B.LACT_ERR_UNSUPPORTED
    assert _call_update(ok, K=None) == B.LACT_ERR_INVALID_ARG
    assert _call_update(ok, n=0) == B.LACT_ERR_INVALID_ARG
    assert _call_update(ok, kvs=10) == B.LACT_ERR_INVALID_ARG
    assert _call_update(ok, es=3) == B.LACT_ERR_INVALID_ARG
    assert _call_update(ok, wsb=16) == B.LACT_ERR_WORKSPACE
    assert _call_update(ok, ws=None) == B.LACT_ERR_WORKSPACE
    assert _call_update(ok, ws=257) == B.LACT_ERR_WORKSPACE
    assert "256-byte" in lib.lact_last_error().decode()
    st = B.LactState(256, 256, 256, None, None, None)
    assert _call_update(L.Config(1, 1, 64, 128, opt="momentum", beta=0.9), st=st) == B.LACT_ERR_INVALID_ARG
    st = B.LactState(256, None, 256, None, None, None)
    assert _call_update(ok, st=st) == B.LACT_ERR_INVALID_ARG


def test_chunked_forward_validation():
    lib = L.load_library()
    c = L.Config(1, 1, 64, 128).to_c()
    s = B.LactState(256, 256, 256, None, None, None)

    def call(T_kv=1024, T_q=1024, ck=256, cq=256, order=0, ws=256, wsb=1 << 30):
        return lib.lact_chunked_forward(ctypes.byref(c), ctypes.byref(s), 256, 256, 256, 256, 256,
                                        T_kv, T_q, ck, cq, order, ws, wsb, None)

    assert call(ck=300) == B.LACT_ERR_INVALID_ARG          # does not divide
    assert call(T_q=512) == B.LACT_ERR_INVALID_ARG         # 4 key chunks vs 2 query chunks
    assert call(order=2) == B.LACT_ERR_INVALID_ARG
    assert call(ck=0) == B.LACT_ERR_INVALID_ARG
    assert call(wsb=0) == B.LACT_ERR_WORKSPACE
    assert "differ" in (lambda: (call(T_q=512), lib.lact_last_error().decode())[1])()


def test_apply_validation():
    lib = L.load_library()
    c = L.Config(1, 1, 64, 128).to_c()
    s = B.LactState(256, 256, 256, None, None, None)
    assert lib.lact_apply(ctypes.byref(c), ctypes.byref(s), 256, None, 4, 256, None, 0, None) == B.LACT_ERR_INVALID_ARG
    assert lib.lact_apply(ctypes.byref(c), ctypes.byref(s), 256, 256, 0, 256, None, 0, None) == B.LACT_ERR_INVALID_ARG
    assert lib.lact_apply(ctypes.byref(c), ctypes.byref(s), 256, 256, 8, 100, None, 0, None) == B.LACT_ERR_INVALID_ARG


def test_products_mode_validation():
    lib = L.load_library()
    c = L.Config(1, 1, 64, 128).to_c()
    c.products = 7
    assert lib.lact_workspace_bytes(ctypes.byref(c), 128, 128) == 0
    s = B.LactState(256, 256, 256, None, None, None)
    assert lib.lact_update(ctypes.byref(c), ctypes.byref(s), 256, 256, 256, 16, 16 * 64, 16, 256,
                           1 << 30, None) == B.LACT_ERR_INVALID_ARG
    assert "products" in lib.lact_last_error().decode()
    assert L.workspace_bytes(L.Config(1, 1, 64, 128, products="split"), 128, 128) > 0


@pytest.mark.parametrize("field", ["norm_mode", "eta_mode"])
def test_variant_mode_validation(field):
    lib = L.load_library()
    c = L.Config(1, 1, 64, 128).to_c()
    setattr(c, field, 5)
    assert lib.lact_workspace_bytes(ctypes.byref(c), 128, 128) == 0
    s = B.LactState(256, 256, 256, None, None, None)
    assert lib.lact_update(ctypes.byref(c), ctypes.byref(s), 256, 256, 256, 16, 16 * 64, 16, 256,
                           1 << 30, None) == B.LACT_ERR_INVALID_ARG
    assert field in lib.lact_last_error().decode()
    ok = L.Config(1, 1, 64, 128, norm="keep", eta_per_matrix=True)
    assert L.workspace_bytes(ok, 128, 128) > 0


def test_binding_checks_the_rate_shape():
    import torch
    K = torch.zeros(1, 2, 16, 64)
    for per_matrix, bad in ((True, (1, 2, 16)), (False, (3, 1, 2, 16))):
        cfg = L.Config(1, 2, 64, 128, eta_per_matrix=per_matrix)
        with pytest.raises(ValueError, match="leading dims"):
            B._check_eta(cfg, torch.zeros(bad), K)


def _forward_rc(cfg, T_kv, chunk_kv, T_q, chunk_q, order=0):
    lib = L.load_library()
    c = cfg.to_c()
    s = B.LactState(256, 256, 256, 256, 256, 256)
    rc = lib.lact_chunked_forward(ctypes.byref(c), ctypes.byref(s), 256, 256, 256, 256, 256, T_kv,
                                  T_q, chunk_kv, chunk_q, order, 256, 1 << 40, None)
    return rc, lib.lact_last_error().decode()


def test_bf16_products_refused_where_muon_amplifies_rounding():
    """bf16 operand products under Muon: refused on chunks of < 1024 keys and on
    runs of more than 4 chunks (the video workload's 14 chunks of 4096); split
    and the default (auto) pass validation there (no GPU here: the first launch
    then fails with a HIP error)."""
    video = dict(T_kv=14 * 4096, chunk_kv=4096, T_q=14 * 4096, chunk_q=4096)
    tiny_chunks = dict(T_kv=300, chunk_kv=100, T_q=21, chunk_q=7)
    for shape, d, h in ((video, 128, 256), (tiny_chunks, 64, 128)):
        rc, msg = _forward_rc(L.Config(1, 2, d, h, opt="muon", products="bf16"), **shape)
        assert rc == B.LACT_ERR_UNSUPPORTED and "1024 keys" in msg, (rc, msg)
        for prod in ("auto", "split"):
            rc, msg = _forward_rc(L.Config(1, 2, d, h, opt="muon", products=prod), **shape)
            assert rc == B.LACT_ERR_HIP, (prod, rc, msg)
    # accepted: one long chunk (posed), four chunks, and every optimizer other than Muon
    for cfg, shape in ((L.Config(1, 2, 64, 128, opt="muon", products="bf16"),
                        dict(T_kv=196608, chunk_kv=196608, T_q=4096, chunk_q=4096)),
                       (L.Config(1, 2, 64, 128, opt="muon", products="bf16"),
                        dict(T_kv=4 * 1024, chunk_kv=1024, T_q=4, chunk_q=1)),
                       (L.Config(1, 2, 64, 128, opt="momentum", beta=0.9, products="bf16"), tiny_chunks),
                       (L.Config(1, 2, 64, 128, opt="gd", products="bf16"), video)):
        rc, msg = _forward_rc(cfg, **shape)
        assert rc == B.LACT_ERR_HIP, (cfg, rc, msg)
    # lact_update counts as one chunk: only the chunk length matters
    cfg = L.Config(1, 1, 64, 128, opt="muon", products="bf16")
    assert _call_update(cfg, n=100) == B.LACT_ERR_UNSUPPORTED
    assert _call_update(cfg, n=1024) == B.LACT_ERR_HIP
    assert _call_update(L.Config(1, 1, 64, 128, opt="muon"), n=100) == B.LACT_ERR_HIP
    # the workspace covers either precision (auto decides per call)
    auto = L.workspace_bytes(L.Config(1, 40, 128, 256, opt="muon"), 4096, 4096)
    for prod in ("bf16", "split"):
        assert auto >= L.workspace_bytes(L.Config(1, 40, 128, 256, opt="muon", products=prod), 4096, 4096)


def _cpu_state(cfg, **override):
    import torch
    st = {}
    for n in ("W1", "W2", "W3") + (("M1", "M2", "M3") if cfg.uses_momentum() else ()):
        shape = (cfg.B, cfg.H, cfg.d, cfg.h) if n[1] == "2" else (cfg.B, cfg.H, cfg.h, cfg.d)
        st[n] = torch.zeros(shape)
    st.update(override)
    return st


def _binding_cases():
    """(entry point, what is wrong) for the binding's shape checks."""
    return ["K d", "V tokens", "eta tokens", "eta per-matrix block", "W2 transposed", "M1 shape",
            "Q batch", "O tokens", "apply Q/O differ", "update K heads"]


@pytest.mark.parametrize("case", _binding_cases())
def test_binding_rejects_mismatched_shapes_before_the_library(case):
    """Every mismatch is a ValueError raised before any library call (CPU
    tensors: with the right shapes the next complaint is about the device)."""
    import torch
    cfg = L.Config(2, 3, 64, 128, opt="momentum", beta=0.9)
    st = _cpu_state(cfg)
    T_kv, T_q = 32, 8
    Q = torch.zeros(2, 3, T_q, 64)
    K = torch.zeros(2, 3, T_kv, 64)
    V = torch.zeros(2, 3, T_kv, 64)
    eta = torch.zeros(2, 3, T_kv)
    O = torch.zeros(2, 3, T_q, 64)
    ws = torch.zeros(16, dtype=torch.uint8)
    fwd = lambda **kw: L.lact_chunked_forward(
        kw.get("cfg", cfg), kw.get("st", st), kw.get("Q", Q), kw.get("K", K), kw.get("V", V),
        kw.get("eta", eta), kw.get("O", O), 16, 4, "apply_then_update", ws)
    call = {
        "K d": lambda: fwd(K=torch.zeros(2, 3, T_kv, 32)),
        "V tokens": lambda: fwd(V=torch.zeros(2, 3, T_kv - 1, 64)),
        "eta tokens": lambda: fwd(eta=torch.zeros(2, 3, T_kv + 1)),
        "eta per-matrix block": lambda: fwd(cfg=L.Config(2, 3, 64, 128, opt="momentum", beta=0.9,
                                                         eta_per_matrix=True)),
        "W2 transposed": lambda: fwd(st=_cpu_state(cfg, W2=torch.zeros(2, 3, 128, 64))),
        "M1 shape": lambda: fwd(st=_cpu_state(cfg, M1=torch.zeros(2, 3, 128, 32))),
        "Q batch": lambda: fwd(Q=torch.zeros(1, 3, T_q, 64)),
        "O tokens": lambda: fwd(O=torch.zeros(2, 3, T_q + 2, 64)),
        "apply Q/O differ": lambda: L.lact_apply(cfg, st, Q, torch.zeros(2, 3, T_q, 64)[:, :, :4],
                                                 m=4, q_stride_bh=T_q * 64),
        "update K heads": lambda: L.lact_update(cfg, st, torch.zeros(2, 2, T_kv, 64), V, eta, ws),
    }[case]
    with pytest.raises(ValueError, match="shape|differ"):
        call()
    # the same call with matching shapes gets past the shape checks
    with pytest.raises(ValueError, match="device tensor"):
        fwd()


def test_linear_net_validation():
    lib = L.load_library()
    ok = L.Config(1, 2, 64, 0, net="linear", norm="none", opt="muon")
    assert L.workspace_bytes(ok, 1000, 100) > 0
    for bad, status, text in ((L.Config(1, 2, 48, 0, net="linear"), B.LACT_ERR_UNSUPPORTED, "d=48"),
                              (L.Config(1, 2, 64, 0, net="linear", eta_per_matrix=True),
                               B.LACT_ERR_UNSUPPORTED, "one rate"),
                              (L.Config(1, 2, 64, 128, norm="none"), B.LACT_ERR_UNSUPPORTED, "linear")):
        c = bad.to_c()
        assert lib.lact_workspace_bytes(ctypes.byref(c), 128, 128) == 0
        s = B.LactState(256, 256, 256, None, None, None)
        assert lib.lact_update(ctypes.byref(c), ctypes.byref(s), 256, 256, 256, 16, 16 * c.d, 16, 256,
                               1 << 30, None) == status
        assert text in lib.lact_last_error().decode()
    c = L.Config(1, 2, 64, 0, net="linear").to_c()
    c.net = 5
    assert lib.lact_workspace_bytes(ctypes.byref(c), 128, 128) == 0
    # the linear state is W1 (and M1) only: W2 / W3 may be NULL
    c = L.Config(1, 2, 64, 0, net="linear", opt="momentum", beta=0.9).to_c()
    assert _call_update(L.Config(1, 2, 64, 0, net="linear", opt="momentum", beta=0.9),
                        st=B.LactState(256, None, None, 256, None, None)) == B.LACT_ERR_HIP
    assert _call_update(L.Config(1, 2, 64, 0, net="linear", opt="momentum", beta=0.9),
                        st=B.LactState(256, None, None, None, None, None)) == B.LACT_ERR_INVALID_ARG


def test_binding_linear_state_shapes():
    import torch
    cfg = L.Config(1, 2, 32, 0, net="linear")
    K = torch.zeros(1, 2, 16, 32)
    eta = torch.zeros(1, 2, 16)
    ws = torch.zeros(16, dtype=torch.uint8)
    with pytest.raises(ValueError, match="W1 has shape"):
        L.lact_update(cfg, {"W1": torch.zeros(1, 2, 32, 16)}, K, K, eta, ws)
    with pytest.raises(ValueError, match="device tensor"):
        L.lact_update(cfg, {"W1": torch.zeros(1, 2, 32, 32)}, K, K, eta, ws)
