"""Causal sliding-window softmax attention in fp64 -- test infrastructure.

Like the rest of ``oracle/``, only tests, the smoke check and the benchmark's
CPU leg may use this module; the library never does.

Source: "LaCT: Test-Time Training Done Right", sections 3.1 and 4: a window
attention computes the relations of tokens within a fixed range; in the
language-model and video configurations it shares Q, K and V with the
large-chunk TTT layer and the two outputs are combined; causality inside a
chunk comes from the causal sliding window.  The pages give neither the window
nor the scale nor the combination, so (readings): query t attends to keys
s with t - window < s <= t, scores q_t . k_s / sqrt(d) by default, a softmax
over those keys, output sum_s p_s v_s; combining = adding to the TTT output.
Written per query with explicit fp64 vector operations.
"""
from __future__ import annotations

import numpy as np


def window_attention(q, k, v, *, window: int, scale=None, q_rows=None):
    """q, k, v [B,H,T,d] -> out [B,H,len(q_rows) or T,d]."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, H, T, d = q.shape
    if window < 1:
        raise ValueError(window)
    sc = 1.0 / np.sqrt(d) if scale is None else float(scale)
    rows = np.arange(T) if q_rows is None else np.asarray(q_rows)
    out = np.zeros((B, H, len(rows), d))
    for b in range(B):
        for h in range(H):
            for i, t in enumerate(rows):
                lo = max(0, t - window + 1)
                s = (k[b, h, lo:t + 1] @ q[b, h, t]) * sc
                p = np.exp(s - np.max(s))
                p /= np.sum(p)
                out[b, h, i] = p @ v[b, h, lo:t + 1]
    return out
