"""The method, as plain float64 definitions.

Sources (DeepSeek-V4 pages):
  * compressor  -- "DeepSeek V4 Attention: Code Reading Map", section "How Does
    Compression Actually Work?" (steps 1-3: load the block's m tokens, softmax
    of the gate scores over the block, weighted sum of the KV rows) and the
    paragraph on the absolute positional encoding added to each token's state.
  * indexer     -- same page, "Aux stream 0 (CSA only)" (per-block scores between
    indexer Q and compressed indexer K, then top-k), with the score
    I = sum_h w_h * ReLU(q_h . k) of the Lightning Indexer.
  * short context -- "DeepSeek V4.1 attention" API page, indexer forward: when
    the candidates number no more than k, every candidate is selected.
  * attention   -- "Code Reading Map", "Phase 3: forward_mqa()" (SWA rows plus
    selected compressed rows, optional sink, one shared KV head) and
    "Concrete Trace" (the window holds the query's own token and the 127 before
    it, and is attended together with the selected compressed entries);
    softmax scale head_dim**-0.5 from the V4.1 page's attention constructor.

Readings where the pages are open (listed in the design notes too):
  * gate granularity: the score half of kv_score has the width of the KV half,
    so the softmax over the block's m tokens runs separately for every channel;
  * the positional encoding [m, d] is added to the gate logits before the softmax;
  * entry i covers positions m*i .. m*i+m-1 and is visible to a query at p
    once its last token is at or before p: n_visible(p) = (p + 1) // m;
  * V equals K: the value of a row is the whole shared d-dim row;
  * top-k ties go to the smaller entry index; selected indices outside
    [0, n_visible(p)) are ignored;
  * a sink adds exp(sink_h) to the softmax denominator only.
"""
from __future__ import annotations

import numpy as np


def n_visible(p: int, m: int) -> int:
    """Compressed entries visible to a query at absolute position p."""
    return (int(p) + 1) // int(m)


def compress(X, S, m: int, ape=None):
    """Compressed entries of a token stream that starts at a block boundary.

    X, S: [T, d] raw KV rows and gate logits. ape: [m, d] or None.
    Returns (C [T//m, d], alpha [T//m, m, d]); a trailing partial block makes no entry.
    """
    X = np.asarray(X, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    T, d = X.shape
    nb = T // m
    z = S[: nb * m].reshape(nb, m, d)
    if ape is not None:
        z = z + np.asarray(ape, dtype=np.float64)[None]
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    alpha = e / e.sum(axis=1, keepdims=True)          # softmax over the block's m tokens, per channel
    C = (alpha * X[: nb * m].reshape(nb, m, d)).sum(axis=1)
    return C, alpha


def index_scores(q, w, K) -> np.ndarray:
    """I[i] = sum_h w[h] * max(0, q[h] . K[i]).  q [H_I, d_I], w [H_I], K [n, d_I] -> [n]."""
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    return np.maximum(K @ q.T, 0.0) @ w


def topk(scores, k: int) -> np.ndarray:
    """The k largest scores' indices, ordered by (-score, index); -1 pads when fewer than k exist."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    order = np.lexsort((np.arange(n), -scores))
    out = np.full(k, -1, dtype=np.int64)
    take = min(k, n)
    out[:take] = order[:take]
    return out


def row_set(p: int, window: int, m: int, selected=None):
    """(sliding-window positions, compressed entry ids) attended by a query at position p.

    selected: the query's top-k ids (CSA) or None for all visible entries (HCA).
    Both parts are kept: a compressed entry and the raw rows it covers can both appear.
    """
    swa = np.arange(max(0, p - window + 1), p + 1, dtype=np.int64)
    nv = n_visible(p, m)
    if selected is None:
        comp = np.arange(nv, dtype=np.int64)
    else:
        sel = np.asarray(selected, dtype=np.int64)
        comp = sel[(sel >= 0) & (sel < nv)]
    return swa, comp


def attention(q, rows, scale: float, sink=None):
    """Single-KV-head attention of every head of q over the shared rows.

    q [H, d], rows [R, d] (K = V = row). sink [H] or None.
    o_h = sum_r e^{l_hr - M} row_r / (sum_r e^{l_hr - M} + e^{sink_h - M}), l = scale * q . row,
    M = max(max_r l_hr, sink_h); lse_h = M + log(denominator).
    With no rows (and no sink) o = 0 and lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64).reshape(-1, q.shape[1])
    H = q.shape[0]
    s = np.full(H, -np.inf) if sink is None else np.asarray(sink, dtype=np.float64)
    if rows.shape[0] == 0:
        lse = s.copy()
        return np.zeros_like(q), lse
    logits = scale * (q @ rows.T)                              # [H, R]
    M = np.maximum(logits.max(axis=1), s)
    p = np.exp(logits - M[:, None])
    den = p.sum(axis=1) + np.exp(s - M)
    o = (p @ rows) / den[:, None]
    return o, M + np.log(den)
