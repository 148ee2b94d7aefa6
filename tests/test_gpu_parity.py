"""GPU parity of the HIP path against the oracle, through the C ABI (MI355X only)."""
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


def _check_step(sc, queries=None, sink=None, split_at=None, check_entries=True):
    """Run the whole step on the GPU and compare every stage with the oracle."""
    wl = sc.wl
    U.say(f"[case] {wl.name} B={len(sc.c_cu) - 1} N={sc.N} max_pos={sc.max_pos()} seed={sc.seed}")
    step, dbg = U.run_step(sc, sink=sink, split_at=split_at)
    qs = list(range(sc.N)) if queries is None else queries
    sink_np = None if sink is None else sink.double().cpu().numpy()
    ref = OP.step(sc, queries=qs, sink=sink_np)
    if check_entries:
        for b in range(len(sc.c_cu) - 1):
            U.check_entries(sc, step, dbg, ref["produced"], b)
    worst = 0.0
    for n_done, t in enumerate(qs):
        if n_done and n_done % 16 == 0:
            U.say(f"[progress] {n_done} of {len(qs)} queries compared")
        if wl.indexer:
            U.check_topk(step.idx[t].cpu().numpy(), step.score[t].cpu().numpy(), ref["topk"][t],
                         ref["scores"][t], wl.topk)
        err, _ = U.check_attention(U.out_np(step, t), ref["o"][t], wl.kv_fmt,
                                   step.lse[t].double().cpu().numpy(), ref["lse"][t])
        worst = max(worst, err)
    # attention alone on the oracle's own selection (identical row sets)
    if wl.indexer:
        sel = torch.full((sc.N, wl.topk), -1, dtype=torch.int32)
        for t in qs:
            sel[t] = torch.from_numpy(ref["topk"][t].astype(np.int32))
        step.attend(sc.q, sc.swa, sc.comp, sc.q_seq, sc.q_pos, sink=sink, topk_idx=sel.to(sc.q.device))
        torch.cuda.synchronize()
        for t in qs:
            U.check_attention(U.out_np(step, t), ref["o"][t], wl.kv_fmt)
    U.say(f"[ok] {wl.name} worst max-abs error {worst:.3e}")
    return step, ref


def test_tiny_csa_full():
    _check_step(G.build(C.TINY_CSA, seed=0, device=_dev()))


def test_tiny_csa_sharp_logits_and_sink():
    sc = G.build(C.TINY_CSA, seed=1, device=_dev(), q_gain=20.0, ape=True)
    sink = torch.tensor([0.0, 2.0, -3.0, float("-inf"), 5.0, 1.0, -1.0, 0.5], device=_dev())
    _check_step(sc, sink=sink)


def test_tiny_csa_compressor_chunking():
    # the stream of 1024 tokens arrives in calls of 1, 5, 250, ... tokens
    sc = G.build(C.TINY_CSA, seed=2, device=_dev())
    _check_step(sc, split_at=[1, 6, 7, 256, 257, 1000])


def test_csa_decode_small_ragged():
    wl = C.CSA_DECODE.with_(B=6, topk=100)
    ctx = [8192, 7001, 4000, 402, 130, 64 * 7 + 3]   # n_visible from 2048 down to 32 (< k)
    sc = G.build(wl, seed=3, device=_dev(), ctx_per_seq=ctx)
    _check_step(sc)


def test_csa_decode_full():
    sc = G.build(C.CSA_DECODE, seed=0, device=_dev())
    _check_step(sc)


def test_hca_decode_small():
    wl = C.HCA_DECODE.with_(B=5)
    sc = G.build(wl, seed=4, device=_dev(), ctx_per_seq=[131072, 65536 + 77, 5000, 127, 129])
    _check_step(sc)


def test_hca_decode_full():
    sc = G.build(C.HCA_DECODE, seed=0, device=_dev())
    _check_step(sc)


def test_hca_three_splits_36_heads_with_sink():
    """96 queries give three splits per query, merged by one wave per head (four heads per
    workgroup, 36 heads: the last workgroup half empty), with a sink; a ragged batch in which some
    queries have no rows in the later splits."""
    wl = C.HCA_DECODE.with_(B=96, H=36)
    rng = np.random.default_rng(34)
    ctx = [131072] + [int(x) for x in rng.integers(1, 131072, size=95)]
    ctx[1:6] = [1, 127, 128, 129, 4096]
    sc = G.build(wl, seed=34, device=_dev(), ctx_per_seq=ctx)
    # three splits: the partials' workspace is N x ceil(H/16) x nsplit x 16 rows of d bf16 + 2 floats
    ws = hcs.sparse_mla_workspace_size(sc.N, wl.H, wl.d, wl.window, wl.m, 0, sc.max_pos())
    assert ws == sc.N * ((wl.H + 15) // 16) * 3 * 16 * (2 * wl.d + 8), ws
    sink = torch.linspace(-1.0, 2.0, wl.H, device=_dev())
    _check_step(sc, sink=sink)


def test_hca_ratio_one_no_window_is_causal_attention():
    """HCA with m=1, window 0 and no top-k is full causal attention (spec invariant)."""
    wl = C.Workload(name="hca_m1", kind="tiny", B=1, ctx=300, H=64, d=512, d_rope=64, m=1, window=0,
                    indexer=False, in_dtype="bf16", n_query=40, q_std=0.5)
    sc = G.build(wl, seed=5, device=_dev())
    step, ref = _check_step(sc)
    X = OP.decode_input(sc.c_x)
    for t in [0, 39]:
        p = int(sc.q_pos[t])
        q = OP.decode_rows("bf16", sc.q[t])
        o_full, _ = OM.attention(q, X[: p + 1], 512 ** -0.5)
        U.check_attention(U.out_np(step, t), o_full, "bf16")


def test_fp8_decode_small():
    wl = C.CSA_DECODE_1M_FP8.with_(B=3, topk=256)
    sc = G.build(wl, seed=6, device=_dev(), ctx_per_seq=[65536, 20000, 900])
    _check_step(sc)


def test_mxfp4_filter_bound_regimes():
    """MXFP4 keys with more than 32768 visible entries (per-wave bounds, filter, select) across
    the regimes of the filter bound: top-2048 over 40000, 33000 + 0 and 140000 entries (kb = 21,
    24 and 6 per 256-entry wave) and top-300 over 100000 entries (more full waves than k: kb = 2).
    A bound above the k-th score would drop selected ids and fail the top-k comparison."""
    wl = C.CSA_DECODE_1M_FP8.with_(B=3)
    sc = G.build(wl, seed=31, device=_dev(), ctx_per_seq=[4 * 40000, 4 * 33000 + 3, 4 * 140000 + 1])
    _check_step(sc)
    wl = C.CSA_DECODE_1M_FP8.with_(B=1, topk=300)
    sc = G.build(wl, seed=32, device=_dev(), ctx_per_seq=[4 * 100000 + 2])
    _check_step(sc)


def test_fp8_decode_1m_full():
    sc = G.build(C.CSA_DECODE_1M_FP8, seed=0, device=_dev())
    _check_step(sc)


def test_prefill_small():
    wl = C.CSA_PREFILL.with_(P0=4096 + 2, Q=300, topk=256)
    sc = G.build(wl, seed=7, device=_dev())
    _check_step(sc, queries=[0, 1, 2, 3, 150, 297, 298, 299])


@pytest.mark.parametrize("fmt", ["fp8ds", "mxfp8"])
def test_prefill_small_quantized_rows(fmt):
    """A prefill chunk over quantized window and compressed rows (fp8_ds, or the V4.1 MXFP8 /
    NVFP4 pair): the head-pair attention with rows dequantised through registers."""
    wl = C.CSA_PREFILL.with_(P0=4096 + 2, Q=300, topk=256, kv_fmt=fmt,
                             comp_fmt="nvfp4" if fmt == "mxfp8" else "")
    sc = G.build(wl, seed=14, device=_dev())
    _check_step(sc, queries=[0, 1, 2, 3, 150, 297, 298, 299])


def test_prefill_long_splits():
    """A query's 1128 rows (18 blocks, the last ragged) in one split of the attention kernel."""
    wl = C.CSA_PREFILL.with_(P0=4096 + 3, Q=256, topk=1000)
    sc = G.build(wl, seed=12, device=_dev())
    _check_step(sc, queries=[0, 1, 100, 254, 255])


def test_prefill_full_sampled():
    """64 of the chunk's 4096 queries, spread over it with both ends: the first queries see the
    prefix only, the last ones the chunk's own 1024 entries as well."""
    sc = G.build(C.CSA_PREFILL, seed=0, device=_dev())
    qs = sorted(set([0, 1, 2, 3] + list(range(67, 4032, 67)) + [4092, 4093, 4094, 4095]))
    assert len(qs) >= 64
    _check_step(sc, queries=qs)


def test_indexer_chunk_matches_per_query_path():
    """hcs_index_topk_chunk scores the queries of one sequence as one matrix product over
    blocks of queries (a ragged last block of queries, a partly visible last block of entries);
    its scores and selections are those of hcs_index_topk with explicit positions, bit for bit."""
    wl = C.CSA_PREFILL.with_(P0=4096 + 2, Q=300, topk=256)
    sc = G.build(wl, seed=11, device=_dev())
    q, qs = U._ix_q_args(sc)
    w = sc.ix_w.contiguous()
    Q, k = w.shape[0], wl.topk
    dev = _dev()
    ia = torch.empty((Q, k), dtype=torch.int32, device=dev)
    ib = torch.empty_like(ia)
    sa = torch.empty((Q, k), dtype=torch.float32, device=dev)
    sb = torch.empty_like(sa)
    hcs.index_topk(q, qs, w, sc.ix, sc.q_seq, sc.q_pos, wl.m, k, wl.P0 + Q - 1, ia, sa)
    hcs.index_topk_chunk(q, qs, w, sc.ix, int(sc.q_seq[0]), wl.P0, wl.m, k, ib, sb)
    torch.cuda.synchronize()
    assert torch.equal(torch.sort(ia, dim=1).values, torch.sort(ib, dim=1).values)
    assert torch.equal(torch.sort(sa, dim=1).values, torch.sort(sb, dim=1).values)


@pytest.mark.parametrize("keys", ["bf16", "mxfp4"])
def test_index_topk_compress_matches_separate_calls(keys):
    """hcs_index_topk_compress (scoring and compressor blocks in one grid) leaves the same
    scores, selections, compressor state and compressed cache as hcs_compress_kv followed by
    hcs_index_topk, bit for bit (ragged batch; some streams end a block at the step, some not;
    MXFP4 keys with fp8_ds rows, one query above 32768 visible entries)."""
    dev = _dev()
    if keys == "bf16":
        wl = C.CSA_DECODE.with_(B=5, topk=96)
        ctx = [1000, 2049, 4096, 3, 777]
    else:
        wl = C.CSA_DECODE_1M_FP8.with_(B=5, topk=300)
        ctx = [1000, 2049, 4 * 40000 + 3, 3, 777]
    sc = G.build(wl, seed=13, device=dev, ctx_per_seq=ctx)
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
    N, k, mp = sc.N, wl.topk, sc.max_pos()
    res = []
    for merged in (False, True):
        sc.comp.pool.copy_(pool0)
        st = state0.clone()
        idx = torch.empty((N, k), dtype=torch.int32, device=dev)
        scr = torch.empty((N, k), dtype=torch.float32, device=dev)
        if merged:
            hcs.index_topk_compress(q, qs, w, sc.ix, sc.q_seq, sc.q_pos, m, k, mp, idx, scr, None,
                                    kv, sco, cu, start, st, sc.comp, m, max_new=1)
        else:
            hcs.compress_kv(kv, sco, cu, start, st, sc.comp, m, max_new=1)
            hcs.index_topk(q, qs, w, sc.ix, sc.q_seq, sc.q_pos, m, k, mp, idx, scr)
        torch.cuda.synchronize()
        res.append((sc.comp.pool.clone(), st, torch.sort(idx, 1).values, torch.sort(scr, 1).values))
    for a, b in zip(res[0], res[1]):
        assert torch.equal(a, b)
    assert not torch.equal(res[0][0], pool0)          # the step did complete some entries


def test_csa_decode_large_selection_ragged():
    """bf16 indexer keys with more than 32768 visible entries (threshold + filter + select path)
    in a ragged batch: a query below 32768 entries, one with fewer entries than k, one at
    position 0 (no compressed entry, a single window row)."""
    wl = C.CSA_DECODE.with_(B=4, topk=300)
    ctx = [4 * 40000, 4 * 33000 + 3, 4 * 250, 1]
    sc = G.build(wl, seed=8, device=_dev(), ctx_per_seq=ctx)
    _check_step(sc)


def test_csa_decode_one_stage_select_up_to_32768():
    """bf16 keys with at most 32768 visible entries take the one-stage select (no filter): keys in
    registers strided over 1024 threads, 16, 24 or 32 per thread (30000, 20000 and 9000 visible
    entries) and contiguous for up to 8192 (5000), top-2048."""
    wl = C.CSA_DECODE.with_(B=4, topk=2048)
    ctx = [4 * 30000, 4 * 20000 + 1, 4 * 9000 + 2, 4 * 5000 + 3]
    sc = G.build(wl, seed=35, device=_dev(), ctx_per_seq=ctx)
    _check_step(sc)


def _tie_case(nv: int, k: int, seed: int):
    """Every indexer key equal, so every score ties: the selection must be the k smallest ids."""
    wl = C.CSA_DECODE.with_(B=2, topk=k)
    sc = G.build(wl, seed=seed, device=_dev(), ctx_per_seq=[4 * nv, 4 * nv + 2])
    pool = sc.ix.pool
    pool.copy_(pool[0:1].expand_as(pool))          # the first page everywhere ...
    row = pool[0, : 2 * wl.d_I].clone()
    pool.view(pool.shape[0], 64, 2 * wl.d_I).copy_(row.view(1, 1, -1).expand(pool.shape[0], 64, -1))  # ... and its first row
    step = PathStep(U.shape_of(sc), device=_dev())
    q, qs = U._ix_q_args(sc)
    step.select(q, qs, sc.ix_w.contiguous(), sc.ix, sc.q_seq, sc.q_pos)
    torch.cuda.synchronize()
    for t in range(2):
        got = np.sort(step.idx[t].cpu().numpy())
        assert np.array_equal(got, np.arange(k)), (nv, k, t, got[:8], got[-8:])
        s = step.score[t].cpu().numpy()
        assert np.all(s == s[0])


def test_topk_ties_go_to_smaller_ids():
    _tie_case(nv=2048, k=512, seed=9)


def test_topk_ties_go_to_smaller_ids_large_selection():
    _tie_case(nv=40000, k=300, seed=10)


def test_empty_batches_launch_nothing():
    """N = 0 (and B = 0) calls succeed without touching any buffer."""
    dev = _dev()
    z32 = torch.zeros(1, dtype=torch.int32, device=dev)
    pool = torch.zeros((1, 64 * 1024), dtype=torch.uint8, device=dev)
    pt = torch.zeros((1, 1), dtype=torch.int32, device=dev)
    cache = hcs.paged(pool, pt, "bf16", 512)
    q = torch.zeros((0, 64, 512), dtype=torch.bfloat16, device=dev)
    out = torch.zeros((0, 64, 512), dtype=torch.bfloat16, device=dev)
    hcs.sparse_mla_decode(q, cache, cache, None, z32[:0], z32[:0], 128, 4, 100, 512 ** -0.5, out)
    st = torch.zeros((0, 3 * 512), dtype=torch.float32, device=dev)
    kv = torch.zeros((0, 512), dtype=torch.bfloat16, device=dev)
    hcs.compress_kv(kv, kv, z32, z32[:0], st, cache, 4, max_new=1)
    torch.cuda.synchronize()
