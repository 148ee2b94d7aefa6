"""Robustness of the HIP path on the GPU, through the C ABI (MI355X only):
  * repeat runs give the same bits (no order of floating-point sums depends on timing);
  * a page-table entry past the pool is reported in the device error word and handled as a
    row that is not resident, while a negative entry is simply "not resident";
  * a selection whose k-th key sits in a radix bin of more than 131072 candidates is exact.
"""
import numpy as np
import pytest
import torch

import hybrid_compressed_sparse_amd as hcs
from hybrid_compressed_sparse_amd.step import PathStep
from oracle import method as OM
from oracle import pipeline as OP
from synth import configs as C
from synth import gen as G

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as U


def _dev():
    return torch.device("cuda:0")


def _fused_step_outputs(sc, step):
    """One CSA decode step with the top-k inside the attention, from the same starting state."""
    wl = sc.wl
    B = len(sc.c_cu) - 1
    state = torch.zeros((B, 3 * wl.d), dtype=torch.float32, device=_dev())
    U.compress_calls(sc, state)
    q, qs = U._ix_q_args(sc)
    step.select(q, qs, sc.ix_w.contiguous(), sc.ix, sc.q_seq, sc.q_pos)
    step.attend(sc.q, sc.swa, sc.comp, sc.q_seq, sc.q_pos)
    torch.cuda.synchronize()
    return step.out.clone(), step.lse.clone(), step.idx.clone()


def test_repeat_runs_bitwise_csa_decode_fused():
    """CSA decode at full size with the selection inside the attention: two runs, same bits of
    out, lse and the selected ids."""
    sc = G.build(C.CSA_DECODE, seed=21, device=_dev())
    U.say(f"[case] repeat runs {sc.wl.name} fused select seed=21")
    step = PathStep(U.shape_of(sc), device=_dev(), select_in_attention=True)
    a = _fused_step_outputs(sc, step)
    b = _fused_step_outputs(sc, step)
    for x, y, name in zip(a, b, ("out", "lse", "ids")):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), name


def test_repeat_runs_bitwise_prefill_chunk():
    """A prefill chunk (indexer chunk kernel, one-stage select, attention in head pairs): two
    runs give the same ids in the same order and the same bits of out and lse."""
    wl = C.CSA_PREFILL.with_(P0=4096 + 2, Q=300, topk=256)
    sc = G.build(wl, seed=22, device=_dev())
    U.say(f"[case] repeat runs {wl.name} Q={wl.Q} seed=22")
    outs = []
    for _ in range(2):
        step, _ = U.run_step(sc)
        outs.append((step.out.clone(), step.lse.clone(), step.idx.clone(), step.score.clone()))
    for x, y, name in zip(outs[0], outs[1], ("out", "lse", "ids", "scores")):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y), name


def test_repeat_runs_two_call_ids_in_ascending_order():
    """The decode select (at most 8192 visible entries, keys in registers) writes the selected
    ids in ascending order, padded with -1: the same order on every run."""
    wl = C.CSA_DECODE.with_(B=4, topk=200)
    sc = G.build(wl, seed=23, device=_dev(), ctx_per_seq=[8192, 6000, 3001, 999])
    U.say(f"[case] ordered ids {wl.name} seed=23")
    runs = []
    for _ in range(2):
        step, _ = U.run_step(sc)
        runs.append(step.idx.clone())
    assert torch.equal(runs[0], runs[1])
    for t in range(4):
        ids = runs[0][t].cpu().numpy()
        v = ids[ids >= 0]
        assert np.all(ids[v.size:] == -1) and np.all(np.diff(v) > 0), t


def test_page_range_error_word():
    """A compressed page-table entry >= num_pages (a corrupt table) makes its rows drop out of
    the attention and sets HCS_DEVERR_PAGE_RANGE; a negative entry drops its rows silently."""
    wl = C.CSA_DECODE.with_(B=2, topk=128)
    sc = G.build(wl, seed=24, device=_dev(), ctx_per_seq=[8192, 4096])
    U.say(f"[case] page range {wl.name} seed=24")
    assert hcs.device_errors(clear=True) == 0
    state = torch.zeros((2, 3 * wl.d), dtype=torch.float32, device=_dev())
    U.compress_calls(sc, state)
    ref = OP.step(sc, queries=[0, 1])
    sel = torch.full((2, wl.topk), -1, dtype=torch.int32)
    for t in range(2):
        sel[t] = torch.from_numpy(ref["topk"][t].astype(np.int32))
    pt = sc.comp.page_table
    npages = sc.comp.pool.shape[0]
    saved = pt.clone()
    bad_page = int(sel[0, 0]) // 64         # a page holding a selected row of query 0
    gone_page = int(sel[1, 0]) // 64        # ... and one of query 1
    step = PathStep(U.shape_of(sc), device=_dev())
    for entry, expect_bit in ((npages + 3, hcs.DEVERR_PAGE_RANGE), (-1, 0)):
        pt.copy_(saved)
        pt[0, bad_page] = entry
        pt[1, gone_page] = entry
        step.attend(sc.q, sc.swa, sc.comp, sc.q_seq, sc.q_pos, topk_idx=sel.to(_dev()))
        bits = hcs.device_errors(clear=True)
        assert bits == expect_bit, (entry, bits)
        for t, page in ((0, bad_page), (1, gone_page)):
            ids = ref["topk"][t]
            kept = ids[(ids // 64) != page]
            assert kept.size < ids.size
            o, lse = OP.query_attention(sc, t, kept, ref["produced"])
            U.check_attention(U.out_np(step, t), o, "bf16", step.lse[t].double().cpu().numpy(), lse)
    pt.copy_(saved)


def _select_with_keys(wl, ctx, seed, mutate):
    """The CSA decode select of one query over keys changed by mutate(keys) (the generated logical
    copy, which the oracle reads, and the pool get the same rows); returns (gpu ids, gpu scores,
    oracle ids, oracle scores)."""
    from synth import layout as SL
    sc = G.build(wl, seed=seed, device=_dev(), ctx_per_seq=[ctx])
    keys = sc.ix.rows[0]
    assert sc.ix.lo[0] == 0
    mutate(keys, sc)
    ids_all = torch.arange(keys.shape[0], device=_dev())
    SL.scatter_rows(sc.ix.pool, sc.ix.fmt, sc.ix.dim, sc.ix.page_table[0], ids_all, keys)
    step = PathStep(U.shape_of(sc), device=_dev())
    q, qs = U._ix_q_args(sc)
    step.select(q, qs, sc.ix_w.contiguous(), sc.ix, sc.q_seq, sc.q_pos)
    torch.cuda.synchronize()
    ids, s = OP.query_topk(sc, 0)
    return step.idx[0].cpu().numpy(), step.score[0].cpu().numpy(), ids, s


def test_select_candidates_clustered_in_one_chunk():
    """The top-2048 of 40000 entries concentrated in one 8192-entry chunk of the filter (3000 keys
    there scaled by 4): that chunk keeps more candidates than the register select loads per
    chunk, so the select finds candidates through the chunks' offsets (keys and ids in LDS)."""
    nv, k = 40000, 2048
    wl = C.CSA_DECODE.with_(B=1, topk=k)
    U.say(f"[case] clustered candidates {wl.name} nv={nv} k={k} seed=26")

    def mutate(keys, sc):
        keys[2 * 8192: 2 * 8192 + 3000] *= 4
    gi, gs, ids, s = _select_with_keys(wl, 4 * nv + 1, 26, mutate)
    in_chunk = ((ids[:k] >= 2 * 8192) & (ids[:k] < 3 * 8192)).sum()
    assert in_chunk > 256, in_chunk                   # that chunk alone holds more than 256 candidates
    U.check_topk(gi, gs, ids, s, k)


def test_select_between_16384_and_32768_candidates():
    """20000 equal keys above every other score among 60000 entries (the best-scoring row doubled,
    exact in bf16): more candidates than the LDS holds with their ids (keys in LDS, ids read
    through the chunk offsets), and the top-300 is the 300 smallest ids of the tie."""
    nv, k = 60000, 300
    wl = C.CSA_DECODE.with_(B=1, topk=k)
    U.say(f"[case] 16384..32768 candidates {wl.name} nv={nv} k={k} seed=27")

    def mutate(keys, sc):
        best = int(OP.query_topk(sc, 0)[0][0])
        keys[:20000] = (keys[best:best + 1] * 2).expand(20000, -1)
    gi, gs, ids, s = _select_with_keys(wl, 4 * nv + 1, 27, mutate)
    assert np.all(s[:20000] == s[0]) and s[0] > s[20000:].max()
    assert np.array_equal(np.sort(gi), np.arange(k))
    U.check_topk(gi, gs, ids, s, k)


def test_select_bin_larger_than_131072():
    """More than 131072 candidates share the k-th key's radix bin (almost every key equal, a few
    slightly larger and smaller): the exact top-k is the larger ones plus the smallest ids of
    the common score."""
    nv, k = 140000, 4096
    wl = C.CSA_DECODE.with_(B=1, topk=k)
    sc = G.build(wl, seed=25, device=_dev(), ctx_per_seq=[4 * nv + 1])
    U.say(f"[case] large bin {wl.name} nv={nv} k={k} seed=25")
    # every key the same row, 100 of them doubled and 100 halved (exact in bf16: scores 2s and
    # s / 2); the generated logical copy (what the oracle reads) and the pool get the same rows
    from synth import layout as SL
    keys = sc.ix.rows[0]
    assert sc.ix.lo[0] == 0 and keys.shape[0] >= nv
    keys.copy_(keys[0:1].expand_as(keys))
    rng = np.random.default_rng(25)
    up = rng.choice(nv, 100, replace=False)
    rest = np.setdiff1d(np.arange(nv), up)
    down = rng.choice(rest, 100, replace=False)
    keys[torch.from_numpy(up).to(_dev())] *= 2
    keys[torch.from_numpy(down).to(_dev())] *= 0.5
    ids_all = torch.arange(keys.shape[0], device=_dev())
    SL.scatter_rows(sc.ix.pool, sc.ix.fmt, sc.ix.dim, sc.ix.page_table[0], ids_all, keys)
    step = PathStep(U.shape_of(sc), device=_dev())
    q, qs = U._ix_q_args(sc)
    step.select(q, qs, sc.ix_w.contiguous(), sc.ix, sc.q_seq, sc.q_pos)
    torch.cuda.synchronize()
    ids, s = OP.query_topk(sc, 0)
    common = np.setdiff1d(rest, down)
    assert np.all(s[common] == s[common[0]]) and s[common[0]] > 0
    assert s[up].min() > s[common[0]] > s[down].max()
    U.check_topk(step.idx[0].cpu().numpy(), step.score[0].cpu().numpy(), ids, s, k)
    assert np.array_equal(np.sort(step.idx[0].cpu().numpy()), np.sort(OM.topk(s, k)))
