"""Dense fp64 attention on logical (never paged) K/V, in NumPy.

TEST INFRASTRUCTURE: pins the C oracle.  It never sees a pool, a block table or
a slot; it takes each sequence's tokens in logical order.  Dense causal attention
as written in "LLM 推理优化的系统视角：从 KV Cache 到调度", section 3.1:
O_t = softmax(Q_t K_{1:t}^T / sqrt(d_h)) V_{1:t}, with the scale passed in.
Grouped heads ("MHA / MQA / GQA", section 4.1 of the same page): query head h
reads kv head h // (Hq // Hkv).
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            return x.to(torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def attention_rows(q, k, v, scale: float) -> np.ndarray:
    """q [Hq, D] attends to all rows of k, v [n, Hkv, D]; returns [Hq, D]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    Hq, D = q.shape
    n, Hkv, _ = k.shape
    G = Hq // Hkv
    out = np.zeros((Hq, D))
    if n == 0:
        return out
    for h in range(Hq):
        g = h // G
        x = scale * (k[:, g, :] @ q[h])
        w = np.exp(x - x.max())
        out[h] = (w @ v[:, g, :]) / w.sum()
    return out


def decode(query, logical_k, logical_v, cu_tokens, scale: float) -> np.ndarray:
    """Each sequence s attends to its tokens cu_tokens[s]:cu_tokens[s+1]."""
    q = _f64(query)
    S = q.shape[0]
    out = np.zeros(q.shape)
    for s in range(S):
        a, b = int(cu_tokens[s]), int(cu_tokens[s + 1])
        out[s] = attention_rows(q[s], logical_k[a:b], logical_v[a:b], scale)
    return out


def causal(q_all, k, v, scale: float) -> np.ndarray:
    """Dense causal attention of a whole sequence: row t sees keys 0..t.
    q_all [n, Hq, D], k/v [n, Hkv, D] -> [n, Hq, D]."""
    q_all = _f64(q_all)
    n = q_all.shape[0]
    out = np.zeros(q_all.shape)
    for t in range(n):
        out[t] = attention_rows(q_all[t], k[: t + 1], v[: t + 1], scale)
    return out


def chunk_rows(q_chunk, k, v, scale: float) -> np.ndarray:
    """Rows of a chunk of length L that ends the sequence k/v of length n:
    row r sits at position n - L + r and sees keys 0..n-L+r."""
    q_chunk = _f64(q_chunk)
    L = q_chunk.shape[0]
    n = k.shape[0]
    out = np.zeros(q_chunk.shape)
    for r in range(L):
        out[r] = attention_rows(q_chunk[r], k[: n - L + r + 1], v[: n - L + r + 1], scale)
    return out
