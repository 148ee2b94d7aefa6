"""One step of the path on device buffers: compress -> (CSA) index + top-k -> sparse attention.

This is the order of a compressed attention layer's step on the DeepSeek-V4 pages ("Code
Reading Map", Phase 2 then Phase 3): the compressor stores the step's completed entries, the
indexer selects compressed entries for each query, and the attention reads both caches. The
class only owns the output and workspace buffers and calls the C entry points in order on the
current stream; no arithmetic happens here. At CSA decode the top-k may instead be taken inside
the attention launch from the indexer's scores (hcs_index_scores_compress, then
hcs_sparse_mla_decode_select): the same selection, one launch fewer.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from . import compress_kv, index_scores_compress, index_topk, index_topk_chunk, index_topk_compress, \
    index_topk_workspace_size, sparse_mla_decode, sparse_mla_decode_select, sparse_mla_prefill_chunk, \
    sparse_mla_prefill_workspace_size, sparse_mla_workspace_size

# most visible entries per query that hcs_sparse_mla_decode_select selects among
SELECT_MAX_VISIBLE = 8192


@dataclass
class StepShape:
    N: int                 # queries
    H: int                 # query heads
    d: int                 # head dim
    m: int                 # compression ratio
    window: int
    max_pos: int           # upper bound of query positions
    topk: int = 0          # 0: HCA (every visible entry)
    prefill: bool = False  # queries are P0 .. P0+N-1 of sequence `seq`
    seq: int = 0
    P0: int = 0


class PathStep:
    """Buffers for one step of a given shape, reused across calls. select_in_attention: at CSA
    decode with d = 512 and bf16 caches, take the top-k inside the attention launch (raises if the
    shape does not allow it)."""

    def __init__(self, shape: StepShape, device="cuda", select_in_attention: bool = False):
        s = self.shape = shape
        self.fused = select_in_attention
        if self.fused and not (s.topk and not s.prefill and s.d == 512
                               and (s.max_pos + 1) // s.m <= SELECT_MAX_VISIBLE):
            raise ValueError("selection inside the attention needs CSA decode, d = 512 and at most "
                             f"{SELECT_MAX_VISIBLE} visible entries")
        self.scores = torch.empty((s.N, (s.max_pos + 1) // s.m), dtype=torch.float32,
                                  device=device) if self.fused else None
        self.out = torch.empty((s.N, s.H, s.d), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((s.N, s.H), dtype=torch.float32, device=device)
        self.idx = torch.empty((s.N, max(s.topk, 1)), dtype=torch.int32, device=device) if s.topk else None
        self.score = torch.empty((s.N, s.topk), dtype=torch.float32, device=device) if s.topk else None
        ix_ws = index_topk_workspace_size(s.N, s.max_pos, s.m, s.topk) if s.topk else 0
        self.ix_ws = torch.empty(max(ix_ws, 1), dtype=torch.uint8, device=device)
        if s.prefill:
            at_ws = sparse_mla_prefill_workspace_size(s.N, s.H, s.d, s.window, s.m, s.topk, s.P0)
        else:
            at_ws = sparse_mla_workspace_size(s.N, s.H, s.d, s.window, s.m, s.topk, s.max_pos)
        self.at_ws = torch.empty(max(at_ws, 1), dtype=torch.uint8, device=device)

    def compress(self, kv, score, cu_new, start_pos, state, comp, max_new, ape=None, dbg=None):
        compress_kv(kv, score, cu_new, start_pos, state, comp, self.shape.m, ape=ape, dbg=dbg,
                    max_new=max_new)

    def select(self, ix_q, ix_q_scale, ix_w, ix_keys, q_seq, q_pos):
        """The indexer: top-k ids into self.idx, or (select_in_attention) the scores only."""
        s = self.shape
        if self.fused:
            index_scores_compress(ix_q, ix_q_scale, ix_w, ix_keys, q_seq, q_pos, s.m, s.max_pos, self.scores)
        elif s.prefill:
            index_topk_chunk(ix_q, ix_q_scale, ix_w, ix_keys, s.seq, s.P0, s.m, s.topk, self.idx,
                             self.score, ws=self.ix_ws)
        else:
            index_topk(ix_q, ix_q_scale, ix_w, ix_keys, q_seq, q_pos, s.m, s.topk, s.max_pos,
                       self.idx, self.score, ws=self.ix_ws)

    def attend(self, q, swa, comp, q_seq=None, q_pos=None, sink=None, topk_idx=None):
        s = self.shape
        idx = topk_idx if topk_idx is not None else self.idx
        if self.fused and topk_idx is None:
            sparse_mla_decode_select(q, swa, comp, self.scores, s.topk, q_seq, q_pos, s.window, s.m,
                                     s.max_pos, s.d ** -0.5, self.out, self.lse, sel_idx=self.idx,
                                     sink=sink, ws=self.at_ws)
        elif s.prefill:
            sparse_mla_prefill_chunk(q, swa, comp, idx, s.seq, s.P0, s.window, s.m, s.d ** -0.5,
                                     self.out, self.lse, sink=sink, ws=self.at_ws)
        else:
            sparse_mla_decode(q, swa, comp, idx, q_seq, q_pos, s.window, s.m, s.max_pos, s.d ** -0.5,
                              self.out, self.lse, sink=sink, ws=self.at_ws)

    def run(self, *, q, swa, comp, q_seq, q_pos, c_kv, c_score, c_cu, c_start, c_state, c_max_new,
            ix_q=None, ix_q_scale=None, ix_w=None, ix_keys=None, ape=None, sink=None,
            dbg: Optional[torch.Tensor] = None):
        """The step, in order on the current stream. At decode the compressor and the indexer
        share one launch (hcs_index_topk_compress: they touch disjoint data); running them on two
        streams instead measured slower inside a captured graph on MI355X, where the cross-stream
        joins cost more than the compressor."""
        s = self.shape
        if self.fused and dbg is None:
            index_scores_compress(ix_q, ix_q_scale, ix_w, ix_keys, q_seq, q_pos, s.m, s.max_pos, self.scores,
                                  c_kv, c_score, c_cu, c_start, c_state, comp, s.m, ape=ape,
                                  max_new=c_max_new)
        elif s.topk and not s.prefill and dbg is None:
            index_topk_compress(ix_q, ix_q_scale, ix_w, ix_keys, q_seq, q_pos, s.m, s.topk, s.max_pos,
                                self.idx, self.score, self.ix_ws, c_kv, c_score, c_cu, c_start, c_state,
                                comp, s.m, ape=ape, max_new=c_max_new)
        else:
            self.compress(c_kv, c_score, c_cu, c_start, c_state, comp, c_max_new, ape=ape, dbg=dbg)
            if s.topk:
                self.select(ix_q, ix_q_scale, ix_w, ix_keys, q_seq, q_pos)
        self.attend(q, swa, comp, q_seq, q_pos, sink=sink)
        return self.out
