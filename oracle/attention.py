"""Naive float64 softmax attention (oracle; test infrastructure only).

What it follows.  The pages fix *what* attention the shared-prefix path must
reproduce: a request that reuses cached prefix KV must get exactly the
attention it would get over its whole, unshared sequence (SGLang paper notes,
section 3: KV cache reuse is valid because a token's KV depends only on the
tokens before it; the vLLM-vs-SGLang page: prefix caching leaves the model's
output unchanged).  The pages do not print the attention formula; the oracle
uses the textbook definition with these readings:
  * scale 1/sqrt(D);
  * a query at absolute position p sees keys 0..p inclusive (a decode token's
    own K/V is stored before it attends, so it sees itself);
  * grouped-query heads: query head h reads KV head floor(h * Hkv / Hq).
Computation: for every query head, scores = scale * q k^T over the request's
full logical key sequence, masked, row-wise max-subtracted exp, normalised,
times V.  No blocking, no online softmax, no merging.
"""
from __future__ import annotations

import numpy as np


def _kv_head(h: int, n_q_heads: int, n_kv_heads: int) -> int:
    return (h * n_kv_heads) // n_q_heads


def attention_probs(q: np.ndarray, k: np.ndarray, q_pos: np.ndarray, scale: float | None = None):
    """Softmax probabilities P [n, Hq, L] (float64) for queries q [n, Hq, D]
    over keys k [L, Hkv, D]; key j is visible to query i iff j <= q_pos[i]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    visible = np.arange(L)[None, :] <= np.asarray(q_pos)[:, None]          # [n, L]
    probs = np.zeros((n, hq, L), np.float64)
    for h in range(hq):
        g = _kv_head(h, hq, hkv)
        s = (q[:, h, :] @ k[:, g, :].T) * scale                             # [n, L]
        s = np.where(visible, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        probs[:, h, :] = e / e.sum(axis=1, keepdims=True)
    return probs


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
                     scale: float | None = None) -> np.ndarray:
    """O [n, Hq, D] (float64).  q [n, Hq, D]; k, v [L, Hkv, D] the request's
    full logical sequence; q_pos [n] absolute positions of the queries."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    n, hq, d = q.shape
    L, hkv, _ = k.shape
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    q_pos = np.asarray(q_pos)
    if n and (q_pos.min() < 0 or q_pos.max() >= L):
        raise ValueError("query position outside the key sequence")
    visible = np.arange(L)[None, :] <= q_pos[:, None]
    out = np.zeros((n, hq, d), np.float64)
    group = hq // hkv
    for g in range(hkv):
        heads = [h for h in range(hq) if _kv_head(h, hq, hkv) == g]
        assert len(heads) == group
        qg = q[:, heads, :].reshape(n * group, d)                           # rows (i, h)
        s = (qg @ k[:, g, :].T) * scale                                     # [n*group, L]
        vis = np.repeat(visible, group, axis=0)
        s = np.where(vis, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=1, keepdims=True)
        out[:, heads, :] = (p @ v[:, g, :]).reshape(n, group, d)
    return out
