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

  * full compressor -- same section, steps 1-7 and "Key design choices": for CSA
    (coff=2) the loaded window is 2m tokens, the block's own m in the primary
    series and the m before it in the overlapping series (the second half of the
    kv / score columns), so boundary tokens feed two entries; then RMSNorm of the
    entry, RoPE on its last 64 dims, and the store.
  * indexer Q/K -- "DeepSeek V4.1 attention" page, `DeepseekV4Indexer` (`forward_q`: RoPE
    and quantization of the projected query, weights times softmax_scale and
    n_head**-0.5; `_produce_k`: k_norm (an RMSNorm) of the projected latent at
    group-boundary tokens, RoPE at the group position, quantization into the key cache;
    `_indexer_k_cache_head_dim`: 68-byte MXFP4 and 132-byte FP8 rows).
  * candidate filtering -- same page, `DeepseekV4Indexer` docstring: besides its own
    top-k, the source layer's indexer lists its best blocks of consecutive compressed
    positions, and a consumer layer restricts its top-k to entries inside the listed
    blocks (readings: a block's score is the max of its entries; entries outside the
    blocks do not take part, and fewer than k taking part are all selected, -1 padded).
  * query preparation and SWA insert -- same page, "Default stream" (the fused
    q-norm / RoPE / KV insert: per-head RMSNorm of the query heads, GPT-J RoPE on
    the last 64 dims of every query head and of the KV row, the KV row stored in
    the sliding-window cache), and the V4.1 page's `_fused_qnorm_rope_kv_insert`
    (the query norm is a switch, with no weight among the op's arguments; the KV
    row is rotated, not normalised, then stored in the cache's format).

Readings where the pages are open (listed in the design notes too):
  * gate granularity: the score half of kv_score has the width of the KV half,
    so the softmax over the block's m tokens runs separately for every channel;
  * the positional encoding [m, d] is added to the gate logits before the softmax;
  * entry i covers positions m*i .. m*i+m-1 and is visible to a query at p
    once its last token is at or before p: n_visible(p) = (p + 1) // m;
  * V equals K: the value of a row is the whole shared d-dim row;
  * top-k ties go to the smaller entry index; selected indices outside
    [0, n_visible(p)) are ignored;
  * a sink adds exp(sink_h) to the softmax denominator only;
  * overlap (coff=2): entry i takes a softmax over 2m logits per channel: block
    i's tokens from the primary series (columns 0..d-1) and block i-1's tokens
    from the overlapping series (columns d..2d-1); entry 0 has only its own m.
    The positional encoding [m, 2d] adds its first half to the primary logits
    and its second half to the overlapping ones, by the token's place in its block;
  * RMSNorm: x / sqrt(mean(x^2) + eps) * weight over the d dims;
  * RoPE: GPT-J style (interleaved pairs (2j, 2j+1)) on the last d_rope dims, at
    the entry's position m*i, with the caller's cos/sin tables [positions, d_rope/2].
  * indexer query / key production (NEXT to the scores): the query's last d_rope dims
    are rotated at the token's position and its weights take softmax_scale * H_I^-0.5;
    a key is RMSNorm (with weight) of the projected latent, rotated at the entry's
    position m*i; both are then quantized to the key cache's format;
  * query norm: over each head's d dims, with no weight (the op takes none); a raw
    token is rotated at its own position p, and its KV row becomes logical row p of
    the sliding-window cache.
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


def compress_overlap(X, S, m: int, ape=None):
    """Compressed entries with the overlapping window (coff = 2).

    X, S: [T, 2d] raw KV rows and gate logits, primary series in columns 0..d-1 and the
    overlapping series in columns d..2d-1. ape: [m, 2d] or None.
    Entry i: per channel c, the softmax over the 2m logits
      S[m*i + j, c] + ape[j, c]              (j < m, block i, primary series)
      S[m*(i-1) + j, d + c] + ape[j, d + c]  (j < m, block i-1, overlapping series; none for i = 0)
    weights the matching raw values X[., c] and X[., d + c].
    Returns (C [T//m, d], alpha [T//m, 2m, d]): alpha[:, :m] weights block i's primary tokens,
    alpha[:, m:] block i-1's overlapping tokens (all zero for entry 0).
    """
    X = np.asarray(X, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    T, d2 = X.shape
    d = d2 // 2
    nb = T // m
    z = S[: nb * m].reshape(nb, m, d2).copy()
    if ape is not None:
        z = z + np.asarray(ape, dtype=np.float64)[None]
    x = X[: nb * m].reshape(nb, m, d2)
    zl = np.full((nb, 2 * m, d), -np.inf)
    xl = np.zeros((nb, 2 * m, d))
    zl[:, :m] = z[:, :, :d]
    xl[:, :m] = x[:, :, :d]
    zl[1:, m:] = z[:-1, :, d:]                       # the previous block, overlapping series
    xl[1:, m:] = x[:-1, :, d:]
    zl = zl - zl.max(axis=1, keepdims=True)
    e = np.exp(zl)
    alpha = e / e.sum(axis=1, keepdims=True)
    C = (alpha * xl).sum(axis=1)
    return C, alpha


def rms_norm(x, weight, eps: float):
    """x / sqrt(mean(x^2) + eps) * weight over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    r = np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return x / r * np.asarray(weight, dtype=np.float64)


def rope_gptj(x, cos, sin, d_rope: int):
    """GPT-J RoPE on the last d_rope dims of each row of x: pair (2j, 2j+1) of those dims
    becomes (a cos_j - b sin_j, a sin_j + b cos_j). cos, sin: [rows, d_rope/2]."""
    x = np.array(x, dtype=np.float64)
    d = x.shape[-1]
    r = x[..., d - d_rope:]
    a, b = r[..., 0::2].copy(), r[..., 1::2].copy()
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    r[..., 0::2] = a * cos - b * sin
    r[..., 1::2] = a * sin + b * cos
    return x


def compress_full(X, S, m: int, coff: int, ape=None, norm_weight=None, eps: float = 1e-6,
                  cos_table=None, sin_table=None, d_rope: int = 0, first_entry: int = 0):
    """The compressor's entries after its epilogue: compress (coff 1) or compress_overlap
    (coff 2), then RMSNorm (when norm_weight is given), then RoPE on the last d_rope dims at
    position m * i (when the tables are given; entry i of this stream is entry first_entry + i
    of its sequence, whose table row is m * (first_entry + i))."""
    C, _ = compress(X, S, m, ape) if coff == 1 else compress_overlap(X, S, m, ape)
    if norm_weight is not None:
        C = rms_norm(C, norm_weight, eps)
    if cos_table is not None and d_rope > 0:
        pos = m * (first_entry + np.arange(C.shape[0]))
        C = rope_gptj(C, np.asarray(cos_table)[pos], np.asarray(sin_table)[pos], d_rope)
    return C


def qnorm_rope(q, pos: int, cos_table, sin_table, d_rope: int, eps: float, q_norm: bool):
    """A raw token's query heads as attention reads them: each head [H, d] normalised to unit
    RMS over its d dims (when q_norm; no weight), then rotated (GPT-J) on its last d_rope dims
    at the token's position pos (row pos of the tables; d_rope 0: no rotation)."""
    q = np.asarray(q, dtype=np.float64)
    if q_norm:
        q = rms_norm(q, np.ones(q.shape[-1]), eps)
    if d_rope > 0:
        c = np.asarray(cos_table, dtype=np.float64)[pos]
        s = np.asarray(sin_table, dtype=np.float64)[pos]
        q = rope_gptj(q, c, s, d_rope)
    return q


def swa_row(kv, pos: int, cos_table, sin_table, d_rope: int):
    """A raw token's KV row [d] as the sliding-window cache holds it (before the cache's own
    rounding): rotated (GPT-J) on its last d_rope dims at the token's position, else as is."""
    kv = np.asarray(kv, dtype=np.float64)
    if d_rope == 0:
        return kv.copy()
    c = np.asarray(cos_table, dtype=np.float64)[pos]
    s = np.asarray(sin_table, dtype=np.float64)[pos]
    return rope_gptj(kv, c, s, d_rope)


def indexer_query(q, pos: int, cos_table, sin_table, d_rope: int, w, softmax_scale: float):
    """Indexer query of a token: q [H_I, d_I] rotated (GPT-J) on its last d_rope dims at the
    token's position; the head weights w [H_I] take the softmax scale and H_I^(-1/2) (both
    positive, so they move no top-k). Returns (q [H_I, d_I], w [H_I])."""
    q = qnorm_rope(q, pos, cos_table, sin_table, d_rope, 0.0, False)
    w = np.asarray(w, dtype=np.float64) * softmax_scale * q.shape[0] ** -0.5
    return q, w


def indexer_key(k_pre, entry: int, m: int, norm_weight, eps: float, cos_table, sin_table,
                d_rope: int):
    """Indexer key of compressed entry `entry`: the projected latent k_pre [d_I] through RMSNorm
    (weight norm_weight) and then GPT-J RoPE on its last d_rope dims at the entry's position
    m * entry, the position the compressor rotates the entry at."""
    k = rms_norm(k_pre, norm_weight, eps)
    if d_rope > 0:
        k = rope_gptj(k, np.asarray(cos_table)[m * entry], np.asarray(sin_table)[m * entry], d_rope)
    return k


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


def candidate_blocks(scores, block: int, n_cand: int) -> np.ndarray:
    """Two-level candidate filtering, source side: the n_cand blocks of `block` consecutive
    entries with the largest block score (the max of the block's entries), ordered by
    (-score, block id); -1 pads when there are fewer blocks."""
    scores = np.asarray(scores, dtype=np.float64)
    nb = -(-scores.shape[0] // block)
    bmax = np.array([scores[b * block:(b + 1) * block].max() for b in range(nb)])
    return topk(bmax, n_cand)


def topk_in_blocks(scores, blocks, block: int, k: int) -> np.ndarray:
    """Two-level candidate filtering, consumer side: the top-k (ties to the smaller id) among
    only the entries of the listed blocks (ids >= 0, each block once); every listed entry is
    selected when there are no more than k of them, and -1 pads."""
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    ids = np.array(sorted(e for b in blocks if b >= 0 for e in range(b * block, min(n, (b + 1) * block))),
                   dtype=np.int64)
    out = np.full(k, -1, dtype=np.int64)
    if ids.size == 0:
        return out
    order = np.lexsort((ids, -scores[ids]))
    sel = ids[order[:k]]
    out[: sel.size] = sel
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
