"""ctypes binding of ``liblact.so`` (include/lact.h), argument marshalling only.

Every step of the layer runs in the library's HIP kernels.  PyTorch only
provides device memory and the current stream.  If the library is missing
the binding raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import dataclasses
import os
from ctypes import c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblact.so")

LACT_OK = 0
LACT_ERR_INVALID_ARG = -1
LACT_ERR_UNSUPPORTED = -2
LACT_ERR_WORKSPACE = -3
LACT_ERR_HIP = -4

LACT_F32, LACT_BF16 = 0, 1
LACT_APPLY_THEN_UPDATE, LACT_UPDATE_THEN_APPLY = 0, 1
LACT_OPT_GD, LACT_OPT_MOMENTUM, LACT_OPT_MUON = 0, 1, 2
PROFILE_PHASES = ("gradient", "tail", "newton_schulz", "step_norm", "apply", "bw_key_tokens", "bw_query_tokens",
                  "bw_contract", "bw_newton_schulz", "window_attention")

ORDER_CODES = {"apply_then_update": LACT_APPLY_THEN_UPDATE, "update_then_apply": LACT_UPDATE_THEN_APPLY}
OPT_CODES = {"gd": LACT_OPT_GD, "momentum": LACT_OPT_MOMENTUM, "muon": LACT_OPT_MUON}
DTYPE_CODES = {"fp32": LACT_F32, "bf16": LACT_BF16}
PRODUCT_CODES = {"bf16": 0, "split": 1, "auto": 2}
NORM_CODES = {"unit": 0, "keep": 1, "none": 2}
NET_CODES = {"swiglu": 0, "linear": 1}

EXPORTED = (
    "lact_config_default", "lact_workspace_bytes", "lact_update", "lact_apply",
    "lact_chunked_forward", "lact_status_string", "lact_last_error", "lact_mfma_path",
    "lact_profile_enable", "lact_profile_read", "lact_version", "lact_chunked_forward_noalloc",
    "lact_noalloc_scratch_bytes", "lact_backward_workspace_bytes", "lact_chunked_backward",
    "lact_window_attention", "lact_block_forward",
)


class LactConfig(ctypes.Structure):
    _fields_ = [
        ("B", c_int32), ("H", c_int32), ("d", c_int32), ("h", c_int32),
        ("io_dtype", c_int32), ("opt", c_int32), ("beta", c_float),
        ("ns_iters", c_int32), ("ns_a", c_float), ("ns_b", c_float), ("ns_c", c_float),
        ("ns_eps", c_float), ("step", c_float), ("norm_eps", c_float), ("products", c_int32),
        ("norm_mode", c_int32), ("eta_mode", c_int32), ("net", c_int32),
    ]


class LactState(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("W1", "W2", "W3", "M1", "M2", "M3")]


class LactGrads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("dQ", "dK", "dV", "deta", "dW1", "dW2", "dW3")]


class LactError(RuntimeError):
    def __init__(self, status, text):
        super().__init__(text)
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load liblact.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                           "(or python chunk_test_amd/build.py)")
    # One HIP runtime per process: PyTorch ships its own copy of the runtime
    # under the same soname.  Loaded first, it is the one the library binds to;
    # loaded after the library, it would start a second runtime beside the
    # library's, and the library's kernel launches would then find no device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.lact_config_default.argtypes = [P(LactConfig)]
    lib.lact_config_default.restype = None
    lib.lact_workspace_bytes.argtypes = [P(LactConfig), c_int64, c_int64]
    lib.lact_workspace_bytes.restype = c_size_t
    lib.lact_update.argtypes = [P(LactConfig), P(LactState), c_void_p, c_void_p, c_void_p,
                                c_int64, c_int64, c_int64, c_void_p, c_size_t, c_void_p]
    lib.lact_update.restype = c_int
    lib.lact_apply.argtypes = [P(LactConfig), P(LactState), c_void_p, c_void_p, c_int64, c_int64,
                               c_void_p, c_size_t, c_void_p]
    lib.lact_apply.restype = c_int
    lib.lact_chunked_forward.argtypes = [P(LactConfig), P(LactState), c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int64,
                                         c_int32, c_void_p, c_size_t, c_void_p]
    lib.lact_chunked_forward.restype = c_int
    lib.lact_chunked_forward_noalloc.argtypes = [P(LactConfig), P(LactState), c_void_p, c_void_p,
                                                 c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                                 c_int64, c_int64, c_int32, c_void_p]
    lib.lact_chunked_forward_noalloc.restype = c_int
    lib.lact_noalloc_scratch_bytes.argtypes = []
    lib.lact_noalloc_scratch_bytes.restype = c_size_t
    lib.lact_backward_workspace_bytes.argtypes = [P(LactConfig), c_int64, c_int64, c_int64]
    lib.lact_backward_workspace_bytes.restype = c_size_t
    lib.lact_chunked_backward.argtypes = [P(LactConfig), P(LactState), c_void_p, c_void_p, c_void_p,
                                          c_void_p, c_void_p, c_void_p, P(LactGrads), c_int64, c_int64,
                                          c_int64, c_int64, c_int32, c_void_p, c_size_t, c_void_p]
    lib.lact_chunked_backward.restype = c_int
    lib.lact_window_attention.argtypes = [P(LactConfig), c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_int64, c_int64, c_float, c_int32, c_void_p]
    lib.lact_window_attention.restype = c_int
    lib.lact_block_forward.argtypes = [P(LactConfig), P(LactState), c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_void_p, c_int64, c_int64, c_int64, c_float, c_int32,
                                       c_void_p, c_size_t, c_void_p]
    lib.lact_block_forward.restype = c_int
    lib.lact_status_string.argtypes = [c_int]
    lib.lact_status_string.restype = c_char_p
    lib.lact_last_error.argtypes = []
    lib.lact_last_error.restype = c_char_p
    lib.lact_mfma_path.argtypes = [c_int32, c_int32, c_int32]
    lib.lact_mfma_path.restype = c_int
    lib.lact_profile_enable.argtypes = [c_int]
    lib.lact_profile_enable.restype = c_int
    lib.lact_profile_read.argtypes = [P(c_double), P(c_int64)]
    lib.lact_profile_read.restype = c_int
    lib.lact_version.argtypes = []
    lib.lact_version.restype = c_int
    _lib = lib
    return lib


def _check(rc: int):
    if rc != LACT_OK:
        lib = load_library()
        raise LactError(rc, f"{lib.lact_status_string(rc).decode()}: {lib.lact_last_error().decode()}")


@dataclasses.dataclass
class Config:
    """Python view of lact_config (defaults as lact_config_default)."""
    B: int
    H: int
    d: int
    h: int
    io_dtype: str = "bf16"
    opt: str = "gd"
    beta: float = 0.0
    ns_iters: int = 5
    ns_a: float = 3.4445
    ns_b: float = -4.7750
    ns_c: float = 2.0315
    ns_eps: float = 1e-7
    step: float = 1.0
    norm_eps: float = 1e-12
    products: str = "auto"  # "auto" | "bf16" | "split" (lact_products)
    norm: str = "unit"  # "unit" | "keep" | "none" (linear net only): row rule after each update
    eta_per_matrix: bool = False  # rates [3,B,H,T]: one per token and matrix (W1, W2, W3)
    net: str = "swiglu"  # "swiglu" | "linear" (state W1 [B,H,d,d] only)

    def to_c(self) -> LactConfig:
        return LactConfig(self.B, self.H, self.d, self.h, DTYPE_CODES[self.io_dtype],
                          OPT_CODES[self.opt], self.beta, self.ns_iters, self.ns_a, self.ns_b,
                          self.ns_c, self.ns_eps, self.step, self.norm_eps,
                          PRODUCT_CODES[self.products], NORM_CODES[self.norm],
                          1 if self.eta_per_matrix else 0, NET_CODES[self.net])

    def uses_momentum(self) -> bool:
        return self.opt == "momentum" or (self.opt == "muon" and self.beta > 0)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _state(st) -> LactState:
    return LactState(*[(_ptr(st.get(n)) if st.get(n) is not None else None)
                       for n in ("W1", "W2", "W3", "M1", "M2", "M3")])


def _stream(stream):
    if stream is not None:
        return c_void_p(stream)
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_tensor(name, t, dtype, device=None, rows_only=False):
    """Device tensor of the given dtype, contiguous (with rows_only: only its
    last dimension dense, for views addressed through explicit strides)."""
    import torch
    if t is None:
        raise ValueError(f"{name} is None")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not (t.stride(-1) == 1 if rows_only else t.is_contiguous()):
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _check_shape(name, t, want, min_last=None):
    """t.shape == want; with min_last, the token axis (the last of eta, -2 of
    the [B,H,T,d] tensors) may instead hold any length >= min_last (views
    into longer sequences)."""
    if t is None:
        raise ValueError(f"{name} is None")
    got, want = tuple(t.shape), tuple(want)
    if min_last is None or len(got) != len(want):
        ok = got == want
    else:
        tok = len(want) - (1 if name == "eta" else 2)
        ok = (all(g == w for i, (g, w) in enumerate(zip(got, want)) if i != tok)
              and got[tok] >= min_last)
    if not ok:
        raise ValueError(f"{name} has shape {got}, expected {want}"
                         + (" (or longer along the tokens)" if min_last is not None else ""))


def _io_dtype(cfg: Config):
    import torch
    return torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32


def _state_shapes(cfg: Config, st):
    """W1, W3 (M1, M3): [B,H,h,d]; W2 (M2): [B,H,d,h].  Linear net: W1 (M1) [B,H,d,d]."""
    if cfg.net == "linear":
        names = ("W1",) + (("M1",) if cfg.uses_momentum() else ())
        for n in names:
            _check_shape(n, st.get(n), (cfg.B, cfg.H, cfg.d, cfg.d))
        return names
    names = ("W1", "W2", "W3") + (("M1", "M2", "M3") if cfg.uses_momentum() else ())
    for n in names:
        want = (cfg.B, cfg.H, cfg.d, cfg.h) if n[1] == "2" else (cfg.B, cfg.H, cfg.h, cfg.d)
        _check_shape(n, st.get(n), want)
    return names


def _check_state(cfg: Config, st):
    import torch
    names = _state_shapes(cfg, st)
    for n in names:
        _check_tensor(n, st[n], torch.float32)
    return [st[n] for n in names]


def _same_device(tensors):
    devs = {t.device for t in tensors if t is not None}
    if len(devs) > 1:
        raise ValueError(f"tensors on several devices: {sorted(str(d) for d in devs)}")


def workspace_bytes(cfg: Config, max_chunk_kv: int, max_chunk_q: int) -> int:
    lib = load_library()
    c = cfg.to_c()
    n = lib.lact_workspace_bytes(ctypes.byref(c), max_chunk_kv, max_chunk_q)
    if n == 0:
        raise LactError(LACT_ERR_UNSUPPORTED, f"no workspace size for {cfg}: "
                        f"{lib.lact_last_error().decode()}")
    return n


def alloc_workspace(cfg: Config, max_chunk_kv: int, max_chunk_q: int, device="cuda"):
    import torch
    return torch.empty(workspace_bytes(cfg, max_chunk_kv, max_chunk_q), dtype=torch.uint8,
                       device=device)


def _eta_shape(cfg: Config, T):
    return ((3,) if cfg.eta_per_matrix else ()) + (cfg.B, cfg.H, T)


def _check_eta(cfg: Config, eta, K, rows_only=False):
    import torch
    want = (3,) + tuple(K.shape[:2]) if cfg.eta_per_matrix else tuple(K.shape[:2])
    if eta is not None and tuple(eta.shape[:-1]) != want:
        raise ValueError(f"eta of shape {tuple(eta.shape)}: leading dims {want} expected")
    _check_tensor("eta", eta, torch.float32, rows_only=rows_only)


def lact_update(cfg: Config, st: dict, K, V, eta, ws, stream=None, n=None,
                kv_stride_bh=None, eta_stride_bh=None):
    """One update on chunk tensors K, V [B,H,n,d] and eta [B,H,n] (per matrix:
    [3,B,H,n]) (in place on st).  With explicit strides the tensors may be
    views into longer sequences (rows dense, pairs and rate blocks at the
    given strides)."""
    lib = load_library()
    views = kv_stride_bh is not None or eta_stride_bh is not None
    n = (K.shape[2] if K is not None and K.dim() == 4 else 0) if n is None else n
    # shapes first: the library cannot see buffer sizes
    _state_shapes(cfg, st)
    for name, t in (("K", K), ("V", V)):
        _check_shape(name, t, (cfg.B, cfg.H, n, cfg.d), min_last=n if views else None)
    _check_shape("eta", eta, _eta_shape(cfg, n), min_last=n if views else None)
    if n < 1:
        raise ValueError(f"n={n} must be >= 1")
    sts = _check_state(cfg, st)
    _check_tensor("K", K, _io_dtype(cfg), rows_only=views)
    _check_tensor("V", V, _io_dtype(cfg), rows_only=views)
    _check_eta(cfg, eta, K, rows_only=views)
    _same_device(sts + [K, V, eta, ws])
    kv_stride_bh = K.shape[2] * cfg.d if kv_stride_bh is None else kv_stride_bh
    eta_stride_bh = eta.shape[-1] if eta_stride_bh is None else eta_stride_bh
    if views:
        # the strides the library is given must be the views' own
        for name, t, inner, ps in (("K", K, cfg.d, kv_stride_bh), ("V", V, cfg.d, kv_stride_bh)):
            if t.stride(2) != inner or t.stride(1) != ps or t.stride(0) != t.shape[1] * ps:
                raise ValueError(f"{name}: strides {t.stride()} do not match kv_stride_bh={ps}")
        lead = eta.dim() - 3  # 1 with a rate block per matrix
        if (eta.stride(-2) != eta_stride_bh or eta.stride(-3) != eta.shape[-2] * eta_stride_bh
                or (lead and eta.stride(0) != eta.shape[1] * eta.shape[2] * eta_stride_bh)):
            raise ValueError(f"eta: strides {eta.stride()} do not match eta_stride_bh={eta_stride_bh}")
    c, s = cfg.to_c(), _state(st)
    _check(lib.lact_update(ctypes.byref(c), ctypes.byref(s), _ptr(K), _ptr(V), _ptr(eta), n,
                           kv_stride_bh, eta_stride_bh, _ptr(ws), ws.numel(), _stream(stream)))


def lact_apply(cfg: Config, st: dict, Q, O, ws=None, stream=None, m=None, q_stride_bh=None):
    """O = f_W(Q) for Q, O [B,H,m,d] (with explicit m and q_stride_bh: the
    first m rows of every pair of contiguous [B,H,T,d] tensors, T >= m)."""
    lib = load_library()
    views = m is not None or q_stride_bh is not None
    m = (Q.shape[2] if Q is not None and Q.dim() == 4 else 0) if m is None else m
    _state_shapes(cfg, st)
    for name, t in (("Q", Q), ("O", O)):
        _check_shape(name, t, (cfg.B, cfg.H, m, cfg.d), min_last=m if views else None)
    if tuple(Q.shape) != tuple(O.shape):
        raise ValueError(f"Q {tuple(Q.shape)} and O {tuple(O.shape)} differ")
    if m < 1:
        raise ValueError(f"m={m} must be >= 1")
    sts = _check_state(cfg, st)
    _check_tensor("Q", Q, _io_dtype(cfg))
    _check_tensor("O", O, _io_dtype(cfg))
    _same_device(sts + [Q, O] + ([ws] if ws is not None else []))
    q_stride_bh = Q.shape[2] * cfg.d if q_stride_bh is None else q_stride_bh
    if q_stride_bh != Q.shape[2] * cfg.d:
        raise ValueError(f"q_stride_bh={q_stride_bh} is not the tensors' pair stride {Q.shape[2] * cfg.d}")
    c, s = cfg.to_c(), _state(st)
    _check(lib.lact_apply(ctypes.byref(c), ctypes.byref(s), _ptr(Q), _ptr(O), m, q_stride_bh,
                          _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def lact_chunked_forward(cfg: Config, st: dict, Q, K, V, eta, O, chunk_kv: int, chunk_q: int,
                         order: str, ws, stream=None):
    """The whole layer over contiguous [B,H,T,d] tensors and eta [B,H,T_kv] (per
    matrix: [3,B,H,T_kv]) (state updated in place)."""
    lib = load_library()
    _state_shapes(cfg, st)
    T_kv = K.shape[2] if K is not None and K.dim() == 4 else -1
    T_q = Q.shape[2] if Q is not None and Q.dim() == 4 else -1
    for name, t, T in (("K", K, T_kv), ("V", V, T_kv), ("Q", Q, T_q), ("O", O, T_q)):
        _check_shape(name, t, (cfg.B, cfg.H, T, cfg.d))
    _check_shape("eta", eta, _eta_shape(cfg, T_kv))
    sts = _check_state(cfg, st)
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O)):
        _check_tensor(name, t, _io_dtype(cfg))
    _check_eta(cfg, eta, K)
    _same_device(sts + [Q, K, V, eta, O, ws])
    c, s = cfg.to_c(), _state(st)
    _check(lib.lact_chunked_forward(ctypes.byref(c), ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V),
                                    _ptr(eta), _ptr(O), T_kv, T_q, chunk_kv, chunk_q,
                                    ORDER_CODES[order], _ptr(ws), ws.numel(), _stream(stream)))


def lact_chunked_forward_noalloc(cfg: Config, st: dict, Q, K, V, eta, O, chunk_kv: int,
                                 chunk_q: int, order: str, stream=None):
    """lact_chunked_forward without a workspace: the library's fixed scratch
    array on the current device (no allocation; overlapping calls on one GPU
    race)."""
    lib = load_library()
    _state_shapes(cfg, st)
    T_kv = K.shape[2] if K is not None and K.dim() == 4 else -1
    T_q = Q.shape[2] if Q is not None and Q.dim() == 4 else -1
    for name, t, T in (("K", K, T_kv), ("V", V, T_kv), ("Q", Q, T_q), ("O", O, T_q)):
        _check_shape(name, t, (cfg.B, cfg.H, T, cfg.d))
    _check_shape("eta", eta, _eta_shape(cfg, T_kv))
    sts = _check_state(cfg, st)
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O)):
        _check_tensor(name, t, _io_dtype(cfg))
    _check_eta(cfg, eta, K)
    _same_device(sts + [Q, K, V, eta, O])
    c, s = cfg.to_c(), _state(st)
    _check(lib.lact_chunked_forward_noalloc(ctypes.byref(c), ctypes.byref(s), _ptr(Q), _ptr(K),
                                            _ptr(V), _ptr(eta), _ptr(O), T_kv, T_q, chunk_kv,
                                            chunk_q, ORDER_CODES[order], _stream(stream)))


def backward_workspace_bytes(cfg: Config, T_kv: int, chunk_kv: int, chunk_q: int) -> int:
    lib = load_library()
    c = cfg.to_c()
    n = lib.lact_backward_workspace_bytes(ctypes.byref(c), T_kv, chunk_kv, chunk_q)
    if n == 0:
        raise LactError(LACT_ERR_UNSUPPORTED, f"no backward workspace size for {cfg}")
    return n


def lact_chunked_backward(cfg: Config, st: dict, Q, K, V, eta, dO, chunk_kv: int, chunk_q: int,
                          order: str, ws=None, dW_final: dict | None = None, stream=None):
    """Cotangents of lact_chunked_forward's inputs given dO (like Q) and,
    optionally, dW_final (cotangents of the final W1, W2, W3).  ``st`` holds
    the initial W1, W2, W3 (not modified).  Returns a dict with dQ, dK, dV
    (like Q, K, V), deta and dW1, dW2, dW3 (new tensors)."""
    import torch
    lib = load_library()
    if cfg.net != "swiglu":
        raise ValueError("backward: SwiGLU fast net only")
    wcfg = dataclasses.replace(cfg, opt="gd", beta=0.0)  # the initial state has no momentum
    _state_shapes(wcfg, st)
    T_kv = K.shape[2] if K is not None and K.dim() == 4 else -1
    T_q = Q.shape[2] if Q is not None and Q.dim() == 4 else -1
    for name, t, T in (("K", K, T_kv), ("V", V, T_kv), ("Q", Q, T_q), ("dO", dO, T_q)):
        _check_shape(name, t, (cfg.B, cfg.H, T, cfg.d))
    _check_shape("eta", eta, _eta_shape(cfg, T_kv))
    if dW_final is not None:
        _state_shapes(wcfg, dW_final)
    sts = _check_state(wcfg, st)
    for name, t in (("Q", Q), ("K", K), ("V", V), ("dO", dO)):
        _check_tensor(name, t, _io_dtype(cfg))
    _check_eta(cfg, eta, K)
    fin = _check_state(wcfg, dW_final) if dW_final is not None else []
    if ws is None:
        ws = torch.empty(backward_workspace_bytes(cfg, T_kv, chunk_kv, chunk_q), dtype=torch.uint8,
                         device=K.device)
    _same_device(sts + fin + [Q, K, V, eta, dO, ws])
    out = {"dQ": torch.empty_like(Q), "dK": torch.empty_like(K), "dV": torch.empty_like(V),
           "deta": torch.empty_like(eta)}
    for n in ("W1", "W2", "W3"):
        out["d" + n] = torch.empty_like(st[n])
    g = LactGrads(*[_ptr(out[n]) for n in ("dQ", "dK", "dV", "deta", "dW1", "dW2", "dW3")])
    c, s = cfg.to_c(), _state(st)
    fs = _state(dW_final) if dW_final is not None else None
    _check(lib.lact_chunked_backward(ctypes.byref(c), ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V),
                                     _ptr(eta), _ptr(dO), ctypes.byref(fs) if fs is not None else None,
                                     ctypes.byref(g), T_kv, T_q, chunk_kv, chunk_q, ORDER_CODES[order],
                                     _ptr(ws), ws.numel(), _stream(stream)))
    return out


def lact_window_attention(cfg: Config, Q, K, V, O, window: int, scale: float = 0.0,
                          accumulate: bool = False, stream=None):
    """O = (or, with accumulate, O +=) causal sliding-window attention of
    Q, K, V [B,H,T,d]; scale <= 0 means 1/sqrt(d)."""
    lib = load_library()
    T = Q.shape[2] if Q is not None and Q.dim() == 4 else -1
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O)):
        _check_shape(name, t, (cfg.B, cfg.H, T, cfg.d))
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O)):
        _check_tensor(name, t, _io_dtype(cfg))
    _same_device([Q, K, V, O])
    c = cfg.to_c()
    _check(lib.lact_window_attention(ctypes.byref(c), _ptr(Q), _ptr(K), _ptr(V), _ptr(O), T, window,
                                     scale, 1 if accumulate else 0, _stream(stream)))


def lact_block_forward(cfg: Config, st: dict, Q, K, V, eta, O, chunk: int, window: int, ws,
                       order: str = "apply_then_update", scale: float = 0.0, stream=None):
    """The LaCT block on shared Q, K, V [B,H,T,d]: O = window attention + the
    TTT layer (chunks of `chunk` keys and queries; state updated in place)."""
    lib = load_library()
    _state_shapes(cfg, st)
    T = K.shape[2] if K is not None and K.dim() == 4 else -1
    for name, t in (("K", K), ("V", V), ("Q", Q), ("O", O)):
        _check_shape(name, t, (cfg.B, cfg.H, T, cfg.d))
    _check_shape("eta", eta, _eta_shape(cfg, T))
    sts = _check_state(cfg, st)
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O)):
        _check_tensor(name, t, _io_dtype(cfg))
    _check_eta(cfg, eta, K)
    _same_device(sts + [Q, K, V, eta, O, ws])
    c, s = cfg.to_c(), _state(st)
    _check(lib.lact_block_forward(ctypes.byref(c), ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V),
                                  _ptr(eta), _ptr(O), T, chunk, window, scale, ORDER_CODES[order],
                                  _ptr(ws), ws.numel(), _stream(stream)))


def noalloc_scratch_bytes() -> int:
    return int(load_library().lact_noalloc_scratch_bytes())


def mfma_path(d: int, h: int, io_dtype: str = "bf16") -> int:
    return load_library().lact_mfma_path(d, h, DTYPE_CODES[io_dtype])


def profile_enable(on: bool):
    _check(load_library().lact_profile_enable(1 if on else 0))


def profile_read():
    """{phase: (total ms, launches)} of the events recorded since the last read."""
    ms = (c_double * len(PROFILE_PHASES))()
    cnt = (c_int64 * len(PROFILE_PHASES))()
    _check(load_library().lact_profile_read(ms, cnt))
    return {p: (ms[i], cnt[i]) for i, p in enumerate(PROFILE_PHASES)}
