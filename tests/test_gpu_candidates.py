"""Two-level candidate filtering on the GPU (hcs_index_topk_cand) against the oracle's
candidate_blocks / topk_in_blocks, over bf16 and MXFP4 indexer keys (MI355X only)."""
import numpy as np
import pytest
import torch

import hybrid_compressed_sparse_amd as hcs
from oracle import method as OM
from oracle import pipeline as OP
from synth import configs as C
from synth import gen as G

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as U


def _dev():
    return torch.device("cuda:0")


def _scenario(kind):
    if kind == "bf16":
        wl = C.CSA_DECODE.with_(B=4, topk=128)
        return G.build(wl, seed=71, device=_dev(), ctx_per_seq=[8192, 3001, 500, 130])
    wl = C.CSA_DECODE_1M_FP8.with_(B=2, topk=256)
    return G.build(wl, seed=72, device=_dev(), ctx_per_seq=[200003, 9000])


def _run(sc, cb, n_cand, cand_in=None):
    q, qs = U._ix_q_args(sc)
    w = sc.ix_w.contiguous()
    N, k = w.shape[0], sc.wl.topk
    dev = _dev()
    out = torch.full((N, k), -7, dtype=torch.int32, device=dev)
    score = torch.empty((N, k), dtype=torch.float32, device=dev)
    cand_out = None if cand_in is not None else torch.full((N, n_cand), -7, dtype=torch.int32, device=dev)
    hcs.index_topk_cand(q, qs, w, sc.ix, sc.q_seq, sc.q_pos, sc.wl.m, k, sc.max_pos(), cb, n_cand, out,
                        cand_in=cand_in, cand_out=cand_out, out_score=score)
    torch.cuda.synchronize()
    return out.cpu().numpy(), score.cpu().numpy(), None if cand_out is None else cand_out.cpu().numpy()


@pytest.mark.parametrize("kind,cb,n_cand", [("bf16", 16, 24), ("bf16", 64, 3), ("mxfp4", 64, 40)])
def test_candidate_source_publishes_top_blocks(kind, cb, n_cand):
    sc = _scenario(kind)
    out, score, cand = _run(sc, cb, n_cand)
    for t in range(sc.N):
        ref_idx, sc_all = OP.query_topk(sc, t)
        U.check_topk(out[t], score[t], ref_idx, sc_all, sc.wl.topk)       # its own top-k is unchanged
        nb = -(-sc_all.shape[0] // cb)
        bmax = np.array([sc_all[b * cb:(b + 1) * cb].max() for b in range(nb)])
        ref_blk = OM.candidate_blocks(sc_all, cb, n_cand)
        g = cand[t]
        U.check_topk(g, np.where(g >= 0, bmax[np.maximum(g, 0)], 0.0), ref_blk, bmax, n_cand)


@pytest.mark.parametrize("kind,cb,n_cand", [("bf16", 16, 24), ("bf16", 32, 2), ("mxfp4", 64, 40)])
def test_candidate_consumer_selects_within_blocks(kind, cb, n_cand):
    sc = _scenario(kind)
    g = torch.Generator().manual_seed(73)
    k = sc.wl.topk
    lists = []
    for t in range(sc.N):
        nv = OM.n_visible(int(sc.q_pos[t]), sc.wl.m)
        nb = -(-nv // cb)
        blk = torch.randperm(max(nb + 3, n_cand), generator=g)[:n_cand].numpy().astype(np.int32)
        blk[::7] = -1                                       # skipped ids; some ids past nv
        lists.append(blk)
    cand_in = torch.from_numpy(np.stack(lists)).to(_dev())
    out, score, _ = _run(sc, cb, n_cand, cand_in)
    for t in range(sc.N):
        _, sc_all = OP.query_topk(sc, t)
        nv = sc_all.shape[0]
        inside = np.array(sorted(e for b in lists[t] if b >= 0 for e in range(b * cb, min(nv, (b + 1) * cb))),
                          dtype=np.int64)
        ref = OM.topk_in_blocks(sc_all, lists[t], cb, k)
        G_ = set(int(i) for i in out[t] if i >= 0)
        O_ = set(int(i) for i in ref if i >= 0)
        assert len(G_) == min(k, inside.size) == int((out[t] >= 0).sum())
        assert G_ <= set(inside.tolist())
        if inside.size > k:
            sk = sc_all[int(ref[k - 1])]
            for i in G_ ^ O_:
                assert abs(sc_all[i] - sk) <= 1e-4 * abs(sk) + 1e-30, (t, i)
        else:
            assert G_ == O_
        sel = out[t] >= 0
        err = np.abs(score[t][sel] - sc_all[out[t][sel]])
        assert err.max(initial=0.0) <= 1e-4 * np.abs(sc_all).max() + 1e-6
