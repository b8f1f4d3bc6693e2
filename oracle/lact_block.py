"""Plain CPU oracle of the LaCT block: causal sliding-window attention beside
the large-chunk TTT layer, on shared queries, keys and values, outputs
summed.

TEST INFRASTRUCTURE ONLY, like ``lact_oracle``: nothing in the product path
may import, call or link this module, and it shares no code with the HIP
library.

Sources ("LaCT: Large Chunk Test-Time Training" review):
* "Local attention and nonlinear memory work together": window attention
  captures local order; the language and video variants can share Q, K and V
  between attention and the TTT layer and add their outputs; in language
  modelling causal sliding-window attention supplies the dependencies
  inside a chunk (the chunk's queries read memory holding only earlier
  chunks).
* "Language modelling: quality and throughput differ": 2,048-token (760M
  model) and 4,096-token (3B model) windows.
* project page, Figure 2 caption: the block's window attention handles the
  structure inside a chunk, the TTT layer the history across chunks.

Readings (the pages give no formula):
* window w: query t attends keys s with t - w < s <= t (w keys including
  itself; causal);
* scores q_t . k_s * scale with scale = 1 / sqrt(d) by default (an
  argument), softmax over the window, output sum_s p_ts v_s;
* the block's output is attention(Q, K, V) + TTT(Q, K, V) with the same
  Q, K, V, the TTT layer in apply-then-update order by default.
"""

from __future__ import annotations

import numpy as np

from . import lact_oracle as F


def window_attention(Q, K, V, window, scale=None):
    """Causal sliding-window attention of one pair: Q, K, V [T, d] -> [T, d]."""
    T, d = Q.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    O = np.zeros_like(Q)
    for t in range(T):
        lo = max(0, t - window + 1)
        s = (K[lo:t + 1] @ Q[t]) * scale
        p = np.exp(s - np.max(s))
        p /= np.sum(p)
        O[t] = p @ V[lo:t + 1]
    return O


def block_forward(state, Q, K, V, eta, chunk, window, hp, order=F.APPLY_THEN_UPDATE, scale=None,
                  dtype=np.float64, pairs=None):
    """The LaCT block over [B, H, T, d] inputs (shared Q, K, V; T_q = T_kv).
    Returns (O, new_state): O = window attention + the TTT layer's output."""
    O_ttt, new = F.lact_chunked_forward(state, Q, K, V, eta, chunk, chunk, order, hp, dtype=dtype,
                                        pairs=pairs)
    B, H = Q.shape[:2]
    todo = [(b, h) for b in range(B) for h in range(H)] if pairs is None else list(pairs)
    O = np.array(O_ttt, copy=True)
    for b, h in todo:
        cast = lambda x: np.asarray(x[b, h], dtype=dtype)
        O[b, h] += window_attention(cast(Q), cast(K), cast(V), window, scale)
    return O, new
