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
PROFILE_PHASES = ("gradient", "tail", "newton_schulz", "step_norm", "apply")

ORDER_CODES = {"apply_then_update": LACT_APPLY_THEN_UPDATE, "update_then_apply": LACT_UPDATE_THEN_APPLY}
OPT_CODES = {"gd": LACT_OPT_GD, "momentum": LACT_OPT_MOMENTUM, "muon": LACT_OPT_MUON}
DTYPE_CODES = {"fp32": LACT_F32, "bf16": LACT_BF16}
PRODUCT_CODES = {"bf16": 0, "split": 1}
NORM_CODES = {"unit": 0, "keep": 1}

EXPORTED = (
    "lact_config_default", "lact_workspace_bytes", "lact_update", "lact_apply",
    "lact_chunked_forward", "lact_status_string", "lact_last_error", "lact_mfma_path",
    "lact_profile_enable", "lact_profile_read", "lact_version",
)


class LactConfig(ctypes.Structure):
    _fields_ = [
        ("B", c_int32), ("H", c_int32), ("d", c_int32), ("h", c_int32),
        ("io_dtype", c_int32), ("opt", c_int32), ("beta", c_float),
        ("ns_iters", c_int32), ("ns_a", c_float), ("ns_b", c_float), ("ns_c", c_float),
        ("ns_eps", c_float), ("step", c_float), ("norm_eps", c_float), ("products", c_int32),
        ("norm_mode", c_int32), ("eta_mode", c_int32),
    ]


class LactState(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("W1", "W2", "W3", "M1", "M2", "M3")]


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
    products: str = "bf16"
    norm: str = "unit"  # "unit" | "keep": updated rows to unit length, or kept at their length
    eta_per_matrix: bool = False  # rates [3,B,H,T]: one per token and matrix (W1, W2, W3)

    def to_c(self) -> LactConfig:
        return LactConfig(self.B, self.H, self.d, self.h, DTYPE_CODES[self.io_dtype],
                          OPT_CODES[self.opt], self.beta, self.ns_iters, self.ns_a, self.ns_b,
                          self.ns_c, self.ns_eps, self.step, self.norm_eps,
                          PRODUCT_CODES[self.products], NORM_CODES[self.norm],
                          1 if self.eta_per_matrix else 0)

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


def _io_dtype(cfg: Config):
    import torch
    return torch.bfloat16 if cfg.io_dtype == "bf16" else torch.float32


def _check_state(cfg: Config, st):
    import torch
    for n in ("W1", "W2", "W3"):
        _check_tensor(n, st[n], torch.float32)
    if cfg.uses_momentum():
        for n in ("M1", "M2", "M3"):
            _check_tensor(n, st.get(n), torch.float32)


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
    _check_state(cfg, st)
    views = kv_stride_bh is not None or eta_stride_bh is not None
    _check_tensor("K", K, _io_dtype(cfg), rows_only=views)
    _check_tensor("V", V, _io_dtype(cfg), rows_only=views)
    _check_eta(cfg, eta, K, rows_only=views)
    n = K.shape[2] if n is None else n
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
        if n > K.shape[2] or n > eta.shape[-1]:
            raise ValueError(f"n={n} beyond the views ({K.shape[2]} keys, {eta.shape[-1]} rates)")
    c, s = cfg.to_c(), _state(st)
    _check(lib.lact_update(ctypes.byref(c), ctypes.byref(s), _ptr(K), _ptr(V), _ptr(eta), n,
                           kv_stride_bh, eta_stride_bh, _ptr(ws), ws.numel(), _stream(stream)))


def lact_apply(cfg: Config, st: dict, Q, O, ws=None, stream=None, m=None, q_stride_bh=None):
    """O = f_W(Q) for Q, O [B,H,m,d]."""
    lib = load_library()
    _check_state(cfg, st)
    _check_tensor("Q", Q, _io_dtype(cfg))
    _check_tensor("O", O, _io_dtype(cfg))
    m = Q.shape[2] if m is None else m
    q_stride_bh = Q.shape[2] * cfg.d if q_stride_bh is None else q_stride_bh
    c, s = cfg.to_c(), _state(st)
    _check(lib.lact_apply(ctypes.byref(c), ctypes.byref(s), _ptr(Q), _ptr(O), m, q_stride_bh,
                          _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)))


def lact_chunked_forward(cfg: Config, st: dict, Q, K, V, eta, O, chunk_kv: int, chunk_q: int,
                         order: str, ws, stream=None):
    """The whole layer over contiguous [B,H,T,d] tensors and eta [B,H,T_kv] (per
    matrix: [3,B,H,T_kv]) (state updated in place)."""
    lib = load_library()
    _check_state(cfg, st)
    for name, t in (("Q", Q), ("K", K), ("V", V), ("O", O)):
        _check_tensor(name, t, _io_dtype(cfg))
    _check_eta(cfg, eta, K)
    c, s = cfg.to_c(), _state(st)
    _check(lib.lact_chunked_forward(ctypes.byref(c), ctypes.byref(s), _ptr(Q), _ptr(K), _ptr(V),
                                    _ptr(eta), _ptr(O), K.shape[2], Q.shape[2], chunk_kv, chunk_q,
                                    ORDER_CODES[order], _ptr(ws), ws.numel(), _stream(stream)))


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
