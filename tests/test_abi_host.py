"""Host-side checks of the C ABI (no GPU needed: nothing here launches a kernel).

* the library loads and exports every function include/lact.h declares;
* workspace sizing;
* argument validation returns the documented status before any HIP call.
"""

import ctypes
import os
import re

import pytest

import chunk_test_amd as L
from chunk_test_amd import lact as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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
