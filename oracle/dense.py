"""Brute-force dense attention in numpy fp64 -- TEST INFRASTRUCTURE ONLY.

Pins the paged C oracle: it takes one sequence's K/V as contiguous arrays (no
pool, no block table, no slot mapping) and writes the attention definition out
with an explicit visibility mask matrix: query i of a chunk that starts after
``context_len`` cached tokens sees keys j <= context_len + i (ngrok, "Serving
models at scale with vLLM", section "Chunked prefill"; "Inside vLLM", section
"Run forward pass", step 3). Query head h reads KV head h // (Hq // Hkv).
"""
from __future__ import annotations

import numpy as np


def visibility_mask(context_len: int, num_queries: int, num_keys: int) -> np.ndarray:
    """mask[i, j] is True when query i (position context_len + i) sees key j."""
    qpos = context_len + np.arange(num_queries)
    return np.arange(num_keys)[None, :] <= qpos[:, None]


def dense_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, context_len: int, scale: float) -> np.ndarray:
    """q [n, Hq, D]; k, v [L, Hkv, D] with L == context_len + n. Returns [n, Hq, D] fp64."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, Hq, D = q.shape
    L, Hkv, _ = k.shape
    assert L == context_len + n and Hq % Hkv == 0
    G = Hq // Hkv
    mask = visibility_mask(context_len, n, L)
    out = np.empty((n, Hq, D))
    for h in range(Hq):
        kh, vh = k[:, h // G, :], v[:, h // G, :]
        logits = float(scale) * (q[:, h, :] @ kh.T)
        logits = np.where(mask, logits, -np.inf)
        w = np.exp(logits - logits.max(axis=1, keepdims=True))
        out[:, h, :] = (w @ vh) / w.sum(axis=1, keepdims=True)
    return out
