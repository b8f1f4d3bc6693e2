"""Seeded synthetic inputs and the named workload configurations.

This module holds no arithmetic of the method: it only draws inputs.  Both
the oracle side (tests, CPU baseline) and the GPU side (tests, bench) take
their inputs from here, so neither depends on the other.

Generator: one numpy ``Generator(PCG64(SeedSequence([seed, tensor_id, b, h])))``
per (tensor, batch, head) block, so every block is reproducible on its own.
tensor_id: W1=0, W3=1, W2=2, Q=3, K=4, V=5, eta=6.  Fast weights are drawn
per head (b = 0) and broadcast over the batch.

Value laws (the workloads' stated distributions):
* W1, W3 ~ N(0, std = 1/sqrt(d)); W2 ~ N(0, std = 1/sqrt(h))  (fan-in scaling).
* q, k, v rows ~ N(0, I_d), each row divided by its L2 norm (in float64),
  then cast to float32 (and, for bf16 workloads, rounded to bfloat16 with
  round-to-nearest-even; the oracle consumes the rounded values).
* eta_i = 0.01 * softplus(z_i), z_i ~ N(0, 1), float32.

The workload shapes follow the pages' settings: 48 images of 512x512 in 8x8
patches = 196,608 tokens; 128 images of 960x536 = 1,029,120 tokens; a 32K
language-model sequence; a ~56K-token video clip as 14 chunks of 4096.
Real tokens would come from trained projections of real data; these
synthetic draws keep the shapes, sizes and norms, not the content.
"""

from __future__ import annotations

import dataclasses

import numpy as np

TENSOR_IDS = {"W1": 0, "W3": 1, "W2": 2, "Q": 3, "K": 4, "V": 5, "eta": 6,
              "eta_W1": 7, "eta_W2": 8, "eta_W3": 9}


def block_rng(seed: int, tensor: str, b: int, h: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence([seed, TENSOR_IDS[tensor], b, h])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16 (ties to even), as float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    nan = np.isnan(x)
    out = r.view(np.float32).copy()
    out[nan] = np.nan
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    h: int
    T_kv: int
    T_q: int
    chunk_kv: int
    chunk_q: int
    order: str            # "apply_then_update" | "update_then_apply"
    opt: str              # "gd" | "momentum" | "muon"
    beta: float = 0.0
    ns_iters: int = 5
    io_dtype: str = "bf16"  # "fp32" | "bf16"
    seed: int = 0
    products: str = "auto"  # "auto" | "bf16" | "split": precision of derived product operands
    norm: str = "unit"      # "unit" | "keep": updated rows to unit length or kept at their length
    eta_per_matrix: bool = False  # rates [3,B,H,T_kv]: one per token and matrix (W1, W2, W3)
    net: str = "swiglu"     # "swiglu" | "linear": f_W(x) = W x with W [d x d] (state W1)

    @property
    def n_chunks(self) -> int:
        return self.T_kv // self.chunk_kv

    @property
    def pairs(self) -> int:
        return self.B * self.H

    def flops(self) -> float:
        """Algorithmic flops of one layer call.

        Per pair and chunk: 12 n d h for the update (two key projections
        4ndh, the value-side product 2ndh, three token contractions 6ndh)
        and 6 m d h for the query read; Muon adds 3 I (4 s^2 l + 2 s^3) per
        pair and update, s = min(d, h), l = max(d, h).
        """
        n, m, d, h = self.chunk_kv, self.chunk_q, self.d, self.h
        if self.net == "linear":
            # dW = U^T K (2 n d^2), O = Q W^T (2 m d^2), Newton-Schulz on d x d
            f = self.pairs * self.n_chunks * (2.0 * n * d * d + 2.0 * m * d * d)
            if self.opt == "muon":
                f += self.pairs * self.n_chunks * 3 * self.ns_iters * 6.0 * d ** 3
            return f
        per_chunk = 12.0 * n * d * h + 6.0 * m * d * h
        f = self.pairs * self.n_chunks * per_chunk
        if self.opt == "muon":
            s, l = min(d, h), max(d, h)
            f += self.pairs * self.n_chunks * 3 * self.ns_iters * (4.0 * s * s * l + 2.0 * s ** 3)
        return f

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 1 sequence, 1 head, d=64, h=128, 1024 tokens in 4 chunks, fp32, GD.
    "tiny": Workload("tiny", B=1, H=1, d=64, h=128, T_kv=1024, T_q=1024,
                     chunk_kv=256, chunk_q=256, order="apply_then_update",
                     opt="gd", io_dtype="fp32"),
    # language-model layer: batch 8, 32768 tokens, 8 heads d=128, h=256,
    # 16 chunks of 2048, apply-then-update, momentum 0.9.
    "lm": Workload("lm", B=8, H=8, d=128, h=256, T_kv=32768, T_q=32768,
                   chunk_kv=2048, chunk_q=2048, order="apply_then_update",
                   opt="momentum", beta=0.9, products="bf16"),
    # posed-image set: 196,608 input tokens as one chunk, 12 heads d=64,
    # h=128, update-then-apply on 4096 query tokens, Muon 5.
    "posed": Workload("posed", B=1, H=12, d=64, h=128, T_kv=196608, T_q=4096,
                      chunk_kv=196608, chunk_q=4096, order="update_then_apply",
                      opt="muon", products="bf16"),
    # AR video: 14 chunks of 4096 tokens, 40 heads d=128, h=256,
    # apply-then-update, Muon 5.
    # (Muon over 14 chunks amplifies bf16 rounding of the gradient's operands
    # from chunk to chunk, so this workload keeps derived operands split)
    "video": Workload("video", B=1, H=40, d=128, h=256, T_kv=57344, T_q=57344,
                      chunk_kv=4096, chunk_q=4096, order="apply_then_update",
                      opt="muon", products="split"),
    # million-token set: 1,029,120 tokens as one chunk, 12 heads d=64, h=128,
    # update-then-apply on 8040 query tokens, Muon 5.
    "million": Workload("million", B=1, H=12, d=64, h=128, T_kv=1029120, T_q=8040,
                        chunk_kv=1029120, chunk_q=8040, order="update_then_apply",
                        opt="muon", products="bf16"),
}


def gen_weights(w: Workload):
    """Initial fast weights, [B,H,h,d] / [B,H,d,h] float32 (drawn per head);
    the linear net's W1 [B,H,d,d] ~ N(0, 1/sqrt(d))."""
    bc = lambda x: np.ascontiguousarray(np.broadcast_to(x[None], (w.B,) + x.shape))
    if w.net == "linear":
        W = np.empty((w.H, w.d, w.d), np.float32)
        for hh in range(w.H):
            W[hh] = block_rng(w.seed, "W1", 0, hh).normal(0.0, 1.0 / np.sqrt(w.d), (w.d, w.d))
        return {"W1": bc(W)}
    W1 = np.empty((w.H, w.h, w.d), np.float32)
    W3 = np.empty((w.H, w.h, w.d), np.float32)
    W2 = np.empty((w.H, w.d, w.h), np.float32)
    for hh in range(w.H):
        W1[hh] = block_rng(w.seed, "W1", 0, hh).normal(0.0, 1.0 / np.sqrt(w.d), (w.h, w.d))
        W3[hh] = block_rng(w.seed, "W3", 0, hh).normal(0.0, 1.0 / np.sqrt(w.d), (w.h, w.d))
        W2[hh] = block_rng(w.seed, "W2", 0, hh).normal(0.0, 1.0 / np.sqrt(w.h), (w.d, w.h))
    return {"W1": bc(W1), "W2": bc(W2), "W3": bc(W3)}


def gen_tokens_block(w: Workload, tensor: str, b: int, hh: int, rows: int) -> np.ndarray:
    """One (b, head) block of q, k or v rows: unit-norm rows, float32 (bf16-rounded)."""
    z = block_rng(w.seed, tensor, b, hh).standard_normal((rows, w.d))
    z /= np.sqrt(np.sum(z * z, axis=1, keepdims=True))
    x = z.astype(np.float32)
    if w.io_dtype == "bf16":
        x = round_bf16(x)
    return x


def gen_eta_block(w: Workload, b: int, hh: int, rows: int, tensor: str = "eta") -> np.ndarray:
    z = block_rng(w.seed, tensor, b, hh).standard_normal(rows)
    return (0.01 * np.logaddexp(0.0, z)).astype(np.float32)


def gen_inputs(w: Workload, heads=None, batches=None):
    """All inputs as float32 numpy arrays [B,H,T,d] (eta [B,H,T_kv], or
    [3,B,H,T_kv] with a rate per token and matrix: three independent draws).

    ``heads`` / ``batches`` optionally restrict generation to some blocks
    (the others are left zero) so that large workloads can be sampled.
    """
    hs = range(w.H) if heads is None else heads
    bs = range(w.B) if batches is None else batches
    Q = np.zeros((w.B, w.H, w.T_q, w.d), np.float32)
    K = np.zeros((w.B, w.H, w.T_kv, w.d), np.float32)
    V = np.zeros((w.B, w.H, w.T_kv, w.d), np.float32)
    eta = np.zeros(((3,) if w.eta_per_matrix else ()) + (w.B, w.H, w.T_kv), np.float32)
    for b in bs:
        for hh in hs:
            Q[b, hh] = gen_tokens_block(w, "Q", b, hh, w.T_q)
            K[b, hh] = gen_tokens_block(w, "K", b, hh, w.T_kv)
            V[b, hh] = gen_tokens_block(w, "V", b, hh, w.T_kv)
            if w.eta_per_matrix:
                for m, t in enumerate(("eta_W1", "eta_W2", "eta_W3")):
                    eta[m, b, hh] = gen_eta_block(w, b, hh, w.T_kv, t)
            else:
                eta[b, hh] = gen_eta_block(w, b, hh, w.T_kv)
    return {"Q": Q, "K": K, "V": V, "eta": eta}
