"""GPU parity of the CSA decode path that selects inside the attention launch
(hcs_index_scores_compress + hcs_sparse_mla_decode_select) against the oracle and against the
two-call path (hcs_index_topk + hcs_sparse_mla_decode), through the C ABI (MI355X only)."""
import numpy as np
import pytest
import torch

import hybrid_compressed_sparse_amd as hcs
from oracle import pipeline as OP
from synth import configs as C
from synth import gen as G

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as U


def _dev():
    return torch.device("cuda:0")


def _scores(sc, aligned=False):
    """Indexer scores of every query over its visible entries (no top-k); rows of nv_cap + 5
    floats, or of a multiple of 64 floats (16-byte aligned rows) when `aligned`."""
    wl = sc.wl
    nv_cap = (sc.max_pos() + 1) // wl.m
    stride = (nv_cap + 63) // 64 * 64 if aligned else nv_cap + 5
    scores = torch.full((sc.N, stride), float("nan"), dtype=torch.float32, device=_dev())
    q, qs = U._ix_q_args(sc)
    hcs.index_scores_compress(q, qs, sc.ix_w.contiguous(), sc.ix, sc.q_seq, sc.q_pos, wl.m, sc.max_pos(),
                              scores)
    return scores


def _select_attend(sc, scores, sink=None):
    wl = sc.wl
    out = torch.empty((sc.N, wl.H, wl.d), dtype=torch.bfloat16, device=_dev())
    lse = torch.empty((sc.N, wl.H), dtype=torch.float32, device=_dev())
    sel = torch.full((sc.N, wl.topk), 7777, dtype=torch.int32, device=_dev())
    hcs.sparse_mla_decode_select(sc.q, sc.swa, sc.comp, scores, wl.topk, sc.q_seq, sc.q_pos, wl.window,
                                 wl.m, sc.max_pos(), wl.d ** -0.5, out, lse, sel_idx=sel, sink=sink)
    return out, lse, sel


def _check(sc, sink=None, aligned=False):
    wl = sc.wl
    U.say(f"[case] select-in-attention {wl.name} N={sc.N} topk={wl.topk} seed={sc.seed}")
    state = torch.zeros((len(sc.c_cu) - 1, 3 * wl.d), dtype=torch.float32, device=_dev())
    U.compress_calls(sc, state)
    scores = _scores(sc, aligned)
    out, lse, sel = _select_attend(sc, scores, sink=sink)
    # the two-call path on the same caches
    idx = torch.empty((sc.N, wl.topk), dtype=torch.int32, device=_dev())
    scr = torch.empty((sc.N, wl.topk), dtype=torch.float32, device=_dev())
    q, qs = U._ix_q_args(sc)
    hcs.index_topk(q, qs, sc.ix_w.contiguous(), sc.ix, sc.q_seq, sc.q_pos, wl.m, wl.topk, sc.max_pos(),
                   idx, scr)
    torch.cuda.synchronize()
    qids = list(range(sc.N))
    sink_np = None if sink is None else sink.double().cpu().numpy()
    ref = OP.step(sc, queries=qids, sink=sink_np)
    worst = 0.0
    for t in qids:
        nv = ref["scores"][t].shape[0]
        s_gpu = scores[t, :nv].double().cpu().numpy()
        s_ref = ref["scores"][t]
        if nv:
            assert np.abs(s_gpu - s_ref).max() <= 1e-4 * max(np.abs(s_ref).max(), 1e-30) + 1e-6
        got = sel[t].cpu().numpy()
        n_sel = min(wl.topk, nv)
        assert np.all(got[n_sel:] == -1), "selected ids are -1 padded"
        assert np.all(np.diff(got[:n_sel]) > 0), "selected ids are in ascending order"
        # the same selection as the indexer's own top-k (same scores, same exact select)
        two = np.sort(idx[t].cpu().numpy())
        assert np.array_equal(np.sort(got), two)
        U.check_topk(got, scores[t].cpu().numpy()[np.maximum(got, 0)], ref["topk"][t], s_ref, wl.topk)
        err, _ = U.check_attention(out[t].float().cpu().numpy().astype(np.float64), ref["o"][t], wl.kv_fmt,
                                   lse[t].double().cpu().numpy(), ref["lse"][t])
        worst = max(worst, err)
    U.say(f"[ok] select-in-attention {wl.name} worst max-abs error {worst:.3e}")


def test_select_in_attention_ragged():
    """Ragged batch: n_visible from 2048 down to fewer than k (every visible entry selected);
    the rows of a query span two splits of the attention."""
    wl = C.CSA_DECODE.with_(B=6, topk=100)
    ctx = [8192, 7001, 4000, 402, 130, 64 * 7 + 3]
    _check(G.build(wl, seed=21, device=_dev(), ctx_per_seq=ctx))
    _check(G.build(wl, seed=27, device=_dev(), ctx_per_seq=ctx), aligned=True)


def test_select_in_attention_csa_decode_full_with_sink():
    """The CSA decode configuration (32 queries, 2048 visible entries, top-512, five splits), with
    score rows of nv_cap + 5 floats and of a multiple of 64 floats."""
    sc = G.build(C.CSA_DECODE, seed=22, device=_dev())
    sink = torch.linspace(-2.0, 3.0, C.CSA_DECODE.H, device=_dev())
    _check(sc, sink=sink)
    _check(sc, sink=sink, aligned=True)


def test_select_in_attention_largest_visible_count():
    """8192 visible entries (the largest the in-attention selection takes) and a short context."""
    wl = C.CSA_DECODE.with_(B=2, topk=256)
    _check(G.build(wl, seed=23, device=_dev(), ctx_per_seq=[4 * 8192, 2]))


def test_select_in_attention_ties_go_to_smaller_ids():
    """Every indexer key equal, so every score ties: the selection is the k smallest ids."""
    k, nv = 512, 2048
    wl = C.CSA_DECODE.with_(B=2, topk=k)
    sc = G.build(wl, seed=24, device=_dev(), ctx_per_seq=[4 * nv, 4 * nv + 2])
    pool = sc.ix.pool
    pool.copy_(pool[0:1].expand_as(pool))
    row = pool[0, : 2 * wl.d_I].clone()
    pool.view(pool.shape[0], 64, 2 * wl.d_I).copy_(row.view(1, 1, -1).expand(pool.shape[0], 64, -1))
    scores = _scores(sc)
    _, _, sel = _select_attend(sc, scores)
    torch.cuda.synchronize()
    for t in range(2):
        assert np.array_equal(sel[t].cpu().numpy(), np.arange(k))


@pytest.mark.parametrize("nv,k", [(2048, 512), (1000, 100)])
def test_select_in_attention_partial_tie_takes_smaller_ids(nv, k):
    """Scores given directly: 100 entries at 2, 300 at 0.5 and the rest tied at 1. The top-k is
    the 100 larger entries and the k - 100 smallest ids of the tie, whose group straddles the
    k-th key."""
    wl = C.CSA_DECODE.with_(B=2, topk=k)
    sc = G.build(wl, seed=26, device=_dev(), ctx_per_seq=[4 * nv, 4 * nv + 3])
    U.say(f"[case] select-in-attention partial tie nv={nv} k={k}")
    nv_cap = (sc.max_pos() + 1) // wl.m
    rng = np.random.default_rng(26)
    s = np.ones((2, nv_cap + 5), dtype=np.float32)
    expect = []
    for t in range(2):
        up = rng.choice(nv, 100, replace=False)
        down = rng.choice(np.setdiff1d(np.arange(nv), up), 300, replace=False)
        s[t, up] = 2.0
        s[t, down] = 0.5
        tie = np.setdiff1d(np.arange(nv), np.concatenate([up, down]))
        expect.append(np.sort(np.concatenate([up, tie[: k - 100]])))
    _, _, sel = _select_attend(sc, torch.from_numpy(s).to(_dev()))
    torch.cuda.synchronize()
    for t in range(2):
        assert np.array_equal(sel[t].cpu().numpy(), expect[t]), t


def test_index_scores_compress_matches_separate_calls():
    """hcs_index_scores_compress with the compressor in the same grid leaves the same scores,
    compressor state and compressed cache as hcs_compress_kv followed by the scores alone,
    bit for bit (ragged batch; some streams end a block at the step, some not)."""
    dev = _dev()
    wl = C.CSA_DECODE.with_(B=5, topk=96)
    sc = G.build(wl, seed=25, device=dev, ctx_per_seq=[1000, 2049, 4096, 3, 777])
    B, d, m = wl.B, wl.d, wl.m
    lens = [sc.c_cu[b + 1] - sc.c_cu[b] for b in range(B)]
    pre = torch.cat([torch.arange(sc.c_cu[b], sc.c_cu[b + 1] - 1, device=dev) for b in range(B)])
    last = torch.tensor([sc.c_cu[b + 1] - 1 for b in range(B)], device=dev)
    state = torch.zeros((B, 3 * d), dtype=torch.float32, device=dev)
    cu_pre = torch.tensor([0] + list(np.cumsum([n - 1 for n in lens])), dtype=torch.int32, device=dev)
    hcs.compress_kv(sc.c_x.index_select(0, pre).contiguous(), sc.c_s.index_select(0, pre).contiguous(),
                    cu_pre, sc.c_start, state, sc.comp, m, max_new=max(lens))
    kv = sc.c_x.index_select(0, last).contiguous()
    sco = sc.c_s.index_select(0, last).contiguous()
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    start = (sc.c_start + torch.tensor([n - 1 for n in lens], dtype=torch.int32, device=dev)).contiguous()
    pool0, state0 = sc.comp.pool.clone(), state.clone()
    q, qs = U._ix_q_args(sc)
    w = sc.ix_w.contiguous()
    nv_cap = (sc.max_pos() + 1) // m
    res = []
    for merged in (False, True):
        sc.comp.pool.copy_(pool0)
        st = state0.clone()
        scores = torch.zeros((sc.N, nv_cap), dtype=torch.float32, device=dev)
        if merged:
            hcs.index_scores_compress(q, qs, w, sc.ix, sc.q_seq, sc.q_pos, m, sc.max_pos(), scores,
                                      kv, sco, cu, start, st, sc.comp, m, max_new=1)
        else:
            hcs.compress_kv(kv, sco, cu, start, st, sc.comp, m, max_new=1)
            hcs.index_scores_compress(q, qs, w, sc.ix, sc.q_seq, sc.q_pos, m, sc.max_pos(), scores)
        torch.cuda.synchronize()
        res.append((sc.comp.pool.clone(), st, scores))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
    assert not torch.equal(res[0][0], pool0)
