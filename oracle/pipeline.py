"""One step of the path for a ``synth`` scenario, in float64, query by query.

Order of the step (DeepSeek-V4 "Code Reading Map", Phase 2 then Phase 3):
  1. the compressor turns every completed block of the step's token stream into
     an entry and stores it in the compressed cache (in the cache's format);
  2. CSA only: the indexer scores every visible compressed entry for each query
     and keeps the top-k;
  3. each query attends to its sliding window plus the selected (CSA) or all
     visible (HCA) compressed entries.
The stored entries of step 1 are what step 3 reads: the oracle rounds its own
float64 entry to the cache format (bf16, or an fp8_ds record) before use.
"""
from __future__ import annotations

import numpy as np
import torch

from . import formats as F
from . import method as M


def _np(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def decode_rows(fmt: str, rows) -> np.ndarray:
    """Stored rows (codes, as the generator made them) -> float64 values."""
    if fmt == "bf16":
        return F.decode_bf16(_np(rows.contiguous().view(torch.int16)).view(np.uint16))
    if fmt == "fp8ds":
        return F.decode_fp8ds(_np(rows.codes), _np(rows.rope.contiguous().view(torch.int16)).view(np.uint16),
                              _np(rows.scales))
    if fmt == "mxfp4":
        return F.decode_mxfp4(_np(rows.codes), _np(rows.scales))
    if fmt == "mxfp8":
        return F.decode_mxfp8(_np(rows.codes), _np(rows.scales))
    if fmt == "nvfp4":
        return F.decode_nvfp4(_np(rows.codes), _np(rows.scales))
    raise ValueError(fmt)


def decode_input(t: torch.Tensor) -> np.ndarray:
    """Compressor inputs (bf16 or float32 tensor) -> float64 values."""
    if t.dtype == torch.bfloat16:
        return F.decode_bf16(_np(t.contiguous().view(torch.int16)).view(np.uint16))
    return _np(t).astype(np.float64)


def store_entry(C: np.ndarray, fmt: str):
    """Round float64 entries to the cache format; returns (decoded stored values, codes)."""
    if fmt == "bf16":
        bits = F.round_bf16(C)
        return F.decode_bf16(bits), bits
    if fmt == "fp8ds":
        rec = F.quantize_fp8ds(C.astype(np.float32))
        return F.decode_fp8ds(*rec), rec
    if fmt == "mxfp8":
        rec = F.quantize_mxfp8(C.astype(np.float32))
        return F.decode_mxfp8(*rec), rec
    if fmt == "nvfp4":
        rec = F.quantize_nvfp4(C.astype(np.float32))
        return F.decode_nvfp4(*rec), rec
    raise ValueError(fmt)


def compress_step(sc):
    """Entries completed by each sequence's compressor stream.

    Returns a list over sequences of (first entry index, C float64 [nb, d], stored float64 [nb, d]).
    """
    m, out = sc.wl.m, []
    ape = None if sc.ape is None else _np(sc.ape).astype(np.float64)
    starts = _np(sc.c_start).tolist()
    for b in range(len(starts)):
        lo, hi = sc.c_cu[b], sc.c_cu[b + 1]
        X = decode_input(sc.c_x[lo:hi])
        S = decode_input(sc.c_s[lo:hi])
        C, _ = M.compress(X, S, m, ape)
        stored, _ = store_entry(C, sc.wl.cfmt) if C.shape[0] else (C, None)
        out.append((starts[b] // m, C, stored))
    return out


def comp_values(sc, b: int, ids: np.ndarray, produced) -> np.ndarray:
    """float64 compressed rows ``ids`` of sequence b, with the step's own entries as stored by it."""
    ids = np.asarray(ids, dtype=np.int64)
    if ids.size == 0:
        return np.zeros((0, sc.wl.d))
    vals = decode_rows(sc.wl.cfmt, sc.comp.logical(b, torch.from_numpy(ids)))
    first, _, stored = produced[b]
    hit = (ids >= first) & (ids < first + stored.shape[0])
    if hit.any():
        vals[hit] = stored[ids[hit] - first]
    return vals


def query_topk(sc, t: int):
    """(top-k ids, scores of all visible entries) of query t."""
    b, p = int(sc.q_seq[t]), int(sc.q_pos[t])
    nv = M.n_visible(p, sc.wl.m)
    q = decode_rows(sc.wl.ix_fmt, _ix_q_row(sc, t))
    w = _np(sc.ix_w[t]).astype(np.float64)
    K = decode_rows(sc.wl.ix_fmt, sc.ix.logical(b, torch.arange(nv))) if nv else np.zeros((0, sc.wl.d_I))
    s = M.index_scores(q, w, K)
    return M.topk(s, sc.wl.topk), s


def _ix_q_row(sc, t):
    if isinstance(sc.ix_q, torch.Tensor):
        return sc.ix_q[t]
    return sc.ix_q.index(t)


def query_attention(sc, t: int, selected, produced, sink=None, scale=None):
    """(o [H, d], lse [H]) of query t over its sliding window and ``selected`` entries (None: all)."""
    wl = sc.wl
    b, p = int(sc.q_seq[t]), int(sc.q_pos[t])
    swa_pos, comp_ids = M.row_set(p, wl.window, wl.m, selected)
    swa_rows = decode_rows(wl.kv_fmt, sc.swa.logical(b, torch.from_numpy(swa_pos))) if swa_pos.size \
        else np.zeros((0, wl.d))
    rows = np.concatenate([swa_rows, comp_values(sc, b, comp_ids, produced)], axis=0)
    q = decode_rows("bf16", sc.q[t])
    return M.attention(q, rows, wl.d ** -0.5 if scale is None else scale, sink)


def step(sc, queries=None, sink=None, selected_override=None):
    """Run the whole step for the given query ids (default: all).

    selected_override: {t: ids} to attend a given selection instead of the oracle's own top-k.
    Returns dict(produced, topk {t: ids}, scores {t: array}, o {t: [H, d]}, lse {t: [H]}).
    """
    produced = compress_step(sc)
    qs = range(sc.N) if queries is None else queries
    res = {"produced": produced, "topk": {}, "scores": {}, "o": {}, "lse": {}}
    for t in qs:
        sel = None
        if sc.wl.indexer:
            ids, s = query_topk(sc, t)
            res["topk"][t], res["scores"][t] = ids, s
            sel = ids
        if selected_override is not None and t in selected_override:
            sel = selected_override[t]
        res["o"][t], res["lse"][t] = query_attention(sc, t, sel, produced, sink)
    return res
