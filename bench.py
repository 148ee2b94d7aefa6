#!/usr/bin/env python
"""Benchmark of one decode step of the hybrid compressed sparse attention path on one MI355X.

A step is the whole hot path over one batch: the compressor on each sequence's new token, the
indexer scores + top-k (CSA) and the sparse MQA attention. Inputs are seeded synthetic tensors
already resident in HBM; the step is captured in a HIP graph over several independent input sets
(rotated, so the 256 MB Infinity Cache cannot serve the caches), replayed, and timed with HIP
events on the capturing stream. One JSON line goes to stdout.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload csa_decode_bf16]

The default run measures the CSA decode workload (the line's value) and, as keys of the same
line, the HCA decode, the 1M-context CSA decode (fp8_ds rows, MXFP4 indexer) and the prefill
chunk, each with per-step percentiles and a roofline entry for its dominant kernel.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode queries/sec and achieved HBM TB/s (% roofline), CSA & HCA layer, 1 GPU"
HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, published


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ algorithmic bytes

def algo_bytes(wl, n_vis: int) -> dict:
    """Bytes one decode step must move per op (the whole batch), by what the method reads/writes.

    attention: q, the window rows, the selected (CSA) or all visible (HCA) compressed rows, the
      top-k ids, the output, lse, and one page-table entry per distinct page touched;
    indexer: the keys of every visible entry, q, w, the selected ids and scores, page tables;
    compressor: read the float32 state (3d), one token's kv and score, write the state and the
      completed entry.
    Score scratch and split partials are not counted: they are this implementation's choice.
    """
    B, H, d = wl.B, wl.H, wl.d
    row_of = {"fp8ds": 584, "mxfp8": 528, "nvfp4": 288}
    row = row_of.get(wl.kv_fmt, 2 * d)                  # window rows
    crow = row_of.get(wl.cfmt, 2 * d)                   # compressed rows
    rows_comp = min(wl.topk, n_vis) if wl.indexer else n_vis
    pt_comp = math.ceil(n_vis / 64) * 4 if not wl.indexer else min(rows_comp, math.ceil(n_vis / 64)) * 4
    attn = B * (H * d * 2                     # q
                + wl.window * row             # sliding window rows
                + rows_comp * crow            # compressed rows
                + (rows_comp * 4 if wl.indexer else 0)
                + H * d * 2 + H * 4           # out, lse
                + 3 * 4 + pt_comp)            # page-table entries
    ix = 0
    if wl.indexer:
        krow = (wl.d_I // 2 + wl.d_I // 32) if wl.ix_fmt == "mxfp4" else 2 * wl.d_I
        qb = wl.H_I * krow
        ix = B * (n_vis * krow + qb + wl.H_I * 4 + wl.topk * 8 + math.ceil(n_vis / 64) * 4)
    in_b = 4 if wl.in_dtype == "f32" else 2
    comp = B * (2 * 3 * d * 4 + 2 * d * in_b + crow)
    return {"attention": attn, "index_topk": ix, "compress": comp, "step": attn + ix + comp}


# ------------------------------------------------------------------ measured HBM traffic

ATTN_SOURCES = ["hybrid_compressed_sparse_amd/csrc/attention.hip", "hybrid_compressed_sparse_amd/csrc/common.h",
                "hybrid_compressed_sparse_amd/csrc/select.h",
                "hybrid_compressed_sparse_amd/csrc/kernels.h"]


def sources_digest(paths) -> str:
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# sources of each op's kernels: a counter summary is used only while they are unchanged
OP_SOURCES = {
    "attention": ATTN_SOURCES,
    "index_topk": ["hybrid_compressed_sparse_amd/csrc/indexer.hip", "hybrid_compressed_sparse_amd/csrc/common.h",
                   "hybrid_compressed_sparse_amd/csrc/select.h", "hybrid_compressed_sparse_amd/csrc/kernels.h",
                   "hybrid_compressed_sparse_amd/csrc/compress_impl.h"],
}


def measured_traffic(workload: str, op: str = "attention"):
    """HBM bytes per launch of `op` from the committed rocprofv3 counter summary
    (profiles/pmc_<op>_<workload>.txt: FETCH_SIZE and WRITE_SIZE per dispatch of each of the
    op's kernels, scaled by the same counters' reading for a copy of known size), or None when
    there is no summary or the op's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"pmc_{op}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("sources_digest") != sources_digest(OP_SOURCES[op]):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def pct_stats(samples) -> dict:
    """p10 / p50 / p90 / mean of per-step times (ms), nearest-rank percentiles."""
    a = sorted(samples)
    if not a:
        return {}

    def pct(p):
        return a[min(len(a) - 1, max(0, math.ceil(p * len(a)) - 1))]
    return {"p10_ms": pct(0.10), "p50_ms": pct(0.50), "p90_ms": pct(0.90), "mean_ms": sum(a) / len(a),
            "samples": len(a)}


# ------------------------------------------------------------------ GPU step

def select_in_attention_ok(wl) -> bool:
    """The CSA decode shapes whose top-k can be taken inside the attention launch."""
    from hybrid_compressed_sparse_amd.step import SELECT_MAX_VISIBLE
    return (wl.kind == "decode" and wl.indexer and wl.d == 512 and wl.kv_fmt == "bf16"
            and wl.cfmt == "bf16" and wl.ctx // wl.m <= SELECT_MAX_VISIBLE)


class Bench:
    def __init__(self, wl, sets: int, seed: int, select_in_attention: bool = False):
        import torch

        from hybrid_compressed_sparse_amd.step import PathStep, StepShape
        from synth import gen as G
        import hybrid_compressed_sparse_amd as hcs

        self.torch, self.hcs = torch, hcs
        self.wl = wl
        dev = torch.device("cuda:0")
        self.sets = []
        for s in range(sets):
            sc = G.build(wl, seed=seed + s, device=dev)
            B, d, m = wl.B, wl.d, wl.m
            state = torch.zeros((B, 3 * d), dtype=torch.float32, device=dev)
            # setup: each stream's tokens before the step's own (the last n_step: one decode
            # token, or the prefill chunk)
            lens = [sc.c_cu[b + 1] - sc.c_cu[b] for b in range(B)]
            ns = [min(sc.n_step, n) for n in lens]
            pre = torch.cat([torch.arange(sc.c_cu[b], sc.c_cu[b + 1] - ns[b], device=dev) for b in range(B)])
            last = torch.cat([torch.arange(sc.c_cu[b + 1] - ns[b], sc.c_cu[b + 1], device=dev) for b in range(B)])
            if pre.numel():
                cu_h = [0]
                for n, k in zip(lens, ns):
                    cu_h.append(cu_h[-1] + n - k)
                cu = torch.tensor(cu_h, dtype=torch.int32, device=dev)
                hcs.compress_kv(sc.c_x.index_select(0, pre).contiguous(),
                                sc.c_s.index_select(0, pre).contiguous(), cu, sc.c_start, state,
                                sc.comp, m, max_new=max(lens))
            cu_s = [0]
            for k in ns:
                cu_s.append(cu_s[-1] + k)
            step_in = dict(
                c_kv=sc.c_x.index_select(0, last).contiguous(),
                c_score=sc.c_s.index_select(0, last).contiguous(),
                c_cu=torch.tensor(cu_s, dtype=torch.int32, device=dev),
                c_start=(sc.c_start + torch.tensor([n - k for n, k in zip(lens, ns)], dtype=torch.int32,
                                                   device=dev)).contiguous(),
                c_state=state, c_max_new=max(ns))
            if wl.indexer:
                if isinstance(sc.ix_q, torch.Tensor):
                    step_in.update(ix_q=sc.ix_q.contiguous(), ix_q_scale=None)
                else:
                    step_in.update(ix_q=sc.ix_q.codes.contiguous(), ix_q_scale=sc.ix_q.scales.contiguous())
                step_in.update(ix_w=sc.ix_w.contiguous(), ix_keys=sc.ix)
            step_in.update(q=sc.q, swa=sc.swa, comp=sc.comp, q_seq=sc.q_seq, q_pos=sc.q_pos)
            self.sets.append((sc, step_in))
            # the logical copies are only needed by the oracle
            sc.comp.rows = sc.swa.rows = None
            if sc.ix is not None:
                sc.ix.rows = None
        sc0 = self.sets[0][0]
        self.step = PathStep(StepShape(N=sc0.N, H=wl.H, d=wl.d, m=wl.m, window=wl.window,
                                       max_pos=sc0.max_pos(), topk=wl.topk if wl.indexer else 0,
                                       prefill=wl.kind == "prefill", seq=0, P0=wl.P0),
                             device=dev, select_in_attention=select_in_attention)
        torch.cuda.synchronize()

    def run_op(self, op: str, i: int):
        sc, a = self.sets[i]
        st = self.step
        if op == "step":
            st.run(**a)
        elif op == "compress":
            st.compress(a["c_kv"], a["c_score"], a["c_cu"], a["c_start"], a["c_state"], a["comp"],
                        a["c_max_new"])
        elif op == "index_topk":
            st.select(a["ix_q"], a["ix_q_scale"], a["ix_w"], a["ix_keys"], a["q_seq"], a["q_pos"])
        elif op == "attention":
            st.attend(a["q"], a["swa"], a["comp"], a["q_seq"], a["q_pos"])

    def graph(self, op: str, sets=None):
        """A HIP graph of `op` over the input sets `sets` (default: all), one launch per set."""
        torch = self.torch
        sets = list(range(len(self.sets))) if sets is None else list(sets)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(2):
                for i in sets:
                    self.run_op(op, i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in sets:
                self.run_op(op, i)
        torch.cuda.synchronize()
        return g

    def distribution(self, op: str, replays: int = 10) -> dict:
        """Percentiles of the time per step of `op` over `replays` replays of the graph of one
        launch per input set (each sample: one replay's HIP-event time / the sets in it, on the
        replay stream), outside the timed region of the headline value."""
        torch = self.torch
        g = self.graph(op)
        g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
        for a, b in ev:
            a.record()
            g.replay()
            b.record()
        torch.cuda.synchronize()
        n = len(self.sets)
        st = pct_stats([a.elapsed_time(b) / n for a, b in ev])
        st["steps_per_sample"] = n
        return st

    def time_graph(self, g, reps: int, warm: int) -> float:
        """Average ms per replay of g over `reps` replays (HIP events on the replay stream)."""
        return self.time_steps([g], reps, warm)

    def time_steps(self, graphs, reps: int, warm: int) -> float:
        """ms for `reps` rounds of replaying `graphs` in order, after `warm` untimed rounds; the
        timed region is bracketed by device synchronisation and HIP events on the replay stream."""
        torch = self.torch
        for _ in range(warm):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            for g in graphs:
                g.replay()
        e1.record()
        e1.synchronize()
        return e0.elapsed_time(e1) / reps


# ------------------------------------------------------------------ CPU baseline (oracle)

def bench_compress_full(wl, sets: int, reps: int) -> dict:
    """The full compressor (overlapping window, RMSNorm, RoPE on 64 dims, bf16 store) at a decode
    step of `wl`: one new token per sequence, each completing an entry. Inputs are seeded random
    values of that shape; the state starts from zeros (the cost does not depend on it)."""
    import torch

    import hybrid_compressed_sparse_amd as hcs
    from synth import gen as G

    dev = torch.device("cuda:0")
    B, d, m, coff, dr = wl.B, wl.d, wl.m, 2, 64
    g = torch.Generator(device="cpu").manual_seed(4242)
    ins = []
    for s in range(sets):
        sc = G.build(wl, seed=3000 + s, device=dev)
        kv = (torch.randn(B, coff * d, generator=g) / d ** 0.5).to(torch.bfloat16).to(dev)
        sco = torch.randn(B, coff * d, generator=g).to(torch.bfloat16).to(dev)
        pos = torch.full((B,), wl.ctx - 1, dtype=torch.int32, device=dev)
        state = torch.zeros((B, 3 * coff * d), dtype=torch.float32, device=dev)
        ins.append((sc, kv, sco, pos, state))
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    w = (torch.rand(d, generator=g) + 0.5).to(dev)
    ang = torch.rand(wl.ctx, dr // 2, generator=g, dtype=torch.float64) * 6.0 - 3.0
    cos, sin = torch.cos(ang).float().to(dev), torch.sin(ang).float().to(dev)

    def run_all():
        for sc, kv, sco, pos, state in ins:
            hcs.compress_kv_full(kv, sco, cu, pos, state, sc.comp, m, coff, norm_weight=w,
                                 rope_cos=cos, rope_sin=sin, max_new=1)

    run_all()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        run_all()
    for _ in range(3):
        gr.replay()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        gr.replay()
    s1.record()
    torch.cuda.synchronize()
    us = s0.elapsed_time(s1) * 1e3 / (reps * sets)
    # bytes the call must move: new rows (kv and score, 2 x 2d bf16), the state read and written
    # (2 x 6d float32), the norm weights, the RoPE rows and the stored entry
    nbytes = B * (2 * coff * d * 2 + 2 * 3 * coff * d * 4 + d * 2 + dr * 4) + d * 4
    del ins
    torch.cuda.empty_cache()
    return {"us_per_call": us, "config": f"B={B}, d={d}, m={m}, coff={coff}, RMSNorm, RoPE {dr} dims, "
            "bf16 store, one token per sequence (each completes an entry)",
            "algorithmic_bytes": nbytes, "gb_s": nbytes / (us * 1e-6) / 1e9}


def bench_insert(wl, n_seq: int, per_seq: int, sets: int, reps: int) -> dict:
    """Query preparation and sliding-window insert (hcs_qnorm_rope_kv_insert: per-head RMSNorm and
    RoPE of the query in place, RoPE of the KV row and its bf16 store) for n_seq sequences of
    `wl`'s shape with per_seq new tokens each, at the end of their context. Inputs are seeded
    random values of that shape, `sets` sets rotated per replay."""
    import torch

    import hybrid_compressed_sparse_amd as hcs
    from synth import layout as SL

    dev = torch.device("cuda:0")
    H, d, dr, ctx = wl.H, wl.d, wl.d_rope, wl.ctx
    N = n_seq * per_seq
    g = torch.Generator(device="cpu").manual_seed(5151)
    p0 = ctx - per_seq
    pg0, pg1 = p0 // 64, (ctx - 1) // 64
    n_pg = pg1 - pg0 + 1
    pt = torch.full((n_seq, (ctx + 63) // 64), -1, dtype=torch.int32)
    for b in range(n_seq):
        pt[b, pg0: pg1 + 1] = torch.arange(b * n_pg, (b + 1) * n_pg, dtype=torch.int32)
    pool = SL.new_pool(n_seq * n_pg, "bf16", d, dev)
    ptd = pt.to(dev)
    swa = hcs.paged(pool, ptd, "bf16", d)
    seq = torch.arange(n_seq, dtype=torch.int32).repeat_interleave(per_seq).to(dev)
    pos = torch.arange(p0, ctx, dtype=torch.int32).repeat(n_seq).to(dev)
    theta = 10000.0 ** (-2.0 * torch.arange(dr // 2, dtype=torch.float64) / dr)
    ang = torch.arange(ctx, dtype=torch.float64)[:, None] * theta[None, :]
    cos, sin = torch.cos(ang).float().to(dev), torch.sin(ang).float().to(dev)
    ins = [(torch.randn(N, H, d, generator=g).to(torch.bfloat16).to(dev),
            (torch.randn(N, d, generator=g) * 0.3).to(torch.bfloat16).to(dev)) for _ in range(sets)]

    def run_all():
        for q, kv in ins:
            hcs.qnorm_rope_kv_insert(q, kv, seq, pos, swa, rope_cos=cos, rope_sin=sin, q_norm=True)

    run_all()
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        run_all()
    for _ in range(2):
        gr.replay()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for _ in range(reps):
        gr.replay()
    s1.record()
    torch.cuda.synchronize()
    us = s0.elapsed_time(s1) * 1e3 / (reps * sets)
    # per token: q read and written (2 x H x d bf16), the KV row read and stored (2 x d bf16),
    # the RoPE row (cos and sin, d_rope/2 float32 each), the token's sequence and position
    per_tok = 2 * H * d * 2 + 2 * d * 2 + dr * 4 + 8
    nbytes = N * per_tok
    gbs = nbytes / (us * 1e-6) / 1e9
    del ins, pool
    torch.cuda.empty_cache()
    return {"us_per_call": us, "tokens": N, "config": f"{n_seq} x {per_seq} tokens, H={H}, d={d}, "
            f"q RMSNorm + RoPE {dr} dims, bf16 SWA rows", "algorithmic_bytes": nbytes, "gb_s": gbs,
            "hbm_frac": gbs / HBM_PEAK_GBS}


def bench_indexer_formats(wl, sets: int, reps: int) -> dict:
    """The indexer (scores + top-k, hcs_index_topk) at `wl`'s shape with keys and queries made by
    hcs_indexer_k_store / hcs_indexer_q_prep from the same seeded values in three formats: bf16,
    MXFP4 (68-byte rows) and FP8 (132-byte rows). Reports each format's time per call (over
    `sets` disjoint groups of sequences, so the keys stream from HBM) and the share of the bf16
    selection that the quantized formats also select. The values are synthetic (normal latents
    through RMSNorm and RoPE), not a trained model's keys."""
    import torch

    import hybrid_compressed_sparse_amd as hcs
    from synth import layout as SL

    dev = torch.device("cuda:0")
    B, H, DI, m, k = wl.B, wl.H_I, wl.d_I, wl.m, wl.topk
    n_vis = wl.ctx // m
    S = sets
    n_seq = B * S
    dr = 64
    g = torch.Generator(device=dev).manual_seed(777)
    theta = 10000.0 ** (-2.0 * torch.arange(dr // 2, dtype=torch.float64) / dr)
    ang = torch.arange(wl.ctx, dtype=torch.float64)[:, None] * theta[None, :]
    cos, sin = torch.cos(ang).float().to(dev), torch.sin(ang).float().to(dev)
    pt = torch.arange(n_seq * ((n_vis + 63) // 64), dtype=torch.int32, device=dev).view(n_seq, -1)
    nw = torch.ones(DI, device=dev)
    caches = {f: SL.new_pool(pt.numel(), f, DI, dev) for f in ("bf16", "mxfp4", "fp8ix")}
    # keys: every entry of every sequence, written in slices of 64 sequences
    for s0 in range(0, n_seq, 64):
        ns = min(64, n_seq - s0)
        k_pre = torch.randn(ns * n_vis, DI, generator=g, device=dev).to(torch.bfloat16)
        ent_seq = torch.arange(s0, s0 + ns, dtype=torch.int32, device=dev).repeat_interleave(n_vis)
        ent_idx = torch.arange(n_vis, dtype=torch.int32, device=dev).repeat(ns)
        for f, pool in caches.items():
            hcs.indexer_k_store(k_pre, ent_seq, ent_idx, m, hcs.paged(pool, pt, f, DI), nw, 1e-6, cos, sin)
        del k_pre, ent_seq, ent_idx
    q = torch.randn(S, B, H, DI, generator=g, device=dev).to(torch.bfloat16)
    w = torch.rand(S, B, H, generator=g, device=dev)
    q_pos = torch.full((B,), wl.ctx - 1, dtype=torch.int32, device=dev)
    q_seq = [torch.arange(i * B, (i + 1) * B, dtype=torch.int32, device=dev) for i in range(S)]
    w_scale = DI ** -0.5 * H ** -0.5
    res = {}
    sel = {}
    for f, pool in caches.items():
        qs, qsc, ws = [], [], []
        for i in range(S):
            if f == "bf16":
                qo, sc = torch.empty(B, H, DI, dtype=torch.bfloat16, device=dev), None
            elif f == "mxfp4":
                qo = torch.empty(B, H, DI // 2, dtype=torch.uint8, device=dev)
                sc = torch.empty(B, H, DI // 32, dtype=torch.uint8, device=dev)
            else:
                qo = torch.empty(B, H, DI, dtype=torch.uint8, device=dev)
                sc = torch.empty(B, H, dtype=torch.float32, device=dev)
            wo = torch.empty(B, H, device=dev)
            hcs.indexer_q_prep(q[i], w[i], q_pos, f, qo, wo, sc, w_scale, cos, sin)
            qs.append(qo)
            qsc.append(sc)
            ws.append(wo)
        paged = hcs.paged(pool, pt, f, DI)
        out = [torch.empty(B, k, dtype=torch.int32, device=dev) for _ in range(S)]
        wsp = torch.empty(hcs.index_topk_workspace_size(B, wl.ctx - 1, m, k), dtype=torch.uint8, device=dev)

        def run_all():
            for i in range(S):
                hcs.index_topk(qs[i], qsc[i], ws[i], paged, q_seq[i], q_pos, m, k, wl.ctx - 1, out[i], ws=wsp)

        run_all()
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            run_all()
        gr.replay()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            gr.replay()
        e1.record()
        torch.cuda.synchronize()
        res[f] = {"us_per_call": e0.elapsed_time(e1) * 1e3 / (reps * S),
                  "key_bytes_per_row": SL.row_bytes(f, DI)}
        sel[f] = torch.stack(out).cpu().numpy()
        del gr, qs, qsc, ws, out, wsp
    ref = sel["bf16"]
    for f in ("mxfp4", "fp8ix"):
        hit = []
        for i in range(S):
            for b in range(B):
                hit.append(len(set(ref[i, b].tolist()) & set(sel[f][i, b].tolist())) / k)
        res[f]["recall_vs_bf16"] = float(sum(hit) / len(hit))
        res[f]["missed_vs_bf16"] = 1.0 - res[f]["recall_vs_bf16"]
        res[f]["speedup_vs_bf16"] = res["bf16"]["us_per_call"] / res[f]["us_per_call"]
    del caches
    torch.cuda.empty_cache()
    res["config"] = (f"{wl.name}: {B} queries per call, {n_vis} visible entries each, top-{k}, "
                     f"H_I={H}, d_I={DI}, {S} disjoint sets of sequences; synthetic values")
    return res


def cpu_info() -> dict:
    """The host's logical CPU count, the CPUs this process may run on, and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    return {"nproc": os.cpu_count(), "affinity_cpus": aff, "cpu_model": model}


def cpu_baseline(wl, seconds: float) -> dict:
    """The oracle (float64 NumPy) timed on this host: whole steps of `wl`'s batch (the
    compressor over every sequence's new token once, then each query's indexer + top-k and
    attention), repeated until `seconds` are spent; queries per second."""
    from threadpoolctl import threadpool_info

    from oracle import pipeline as OP
    from synth import gen as G

    sc = G.build(wl, seed=0, device="cpu")
    OP.step(sc, queries=[0])                      # warm the caches of the decoders
    t0 = time.perf_counter()
    steps = 0
    while steps == 0 or time.perf_counter() - t0 < seconds:
        OP.step(sc)
        steps += 1
    dt = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": steps * sc.N / dt, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{steps} whole steps of {wl.name} ({sc.N} queries each: compressor over the batch's "
                      f"new tokens, per query indexer + top-k and attention), float64 NumPy with "
                      f"{threads} BLAS threads, {dt:.1f} s",
            **cpu_info()}


# ------------------------------------------------------------------ prefill chunk

BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16, published


def prefill_flops(wl) -> dict:
    """MFMA work of one prefill chunk: the indexer's q.k over every visible entry of every query
    (2 flops per multiply-add), attention's S = q k^T and O = P V over each query's rows."""
    ix = at = 0
    for j in range(wl.Q):
        p = wl.P0 + j
        nv = (p + 1) // wl.m
        rows = min(wl.window, p + 1) + (min(wl.topk, nv) if wl.indexer else nv)
        ix += 2 * nv * wl.H_I * wl.d_I if wl.indexer else 0
        at += 2 * 2 * rows * wl.H * wl.d
    return {"index_topk": ix, "attention": at, "step": ix + at}


def measure_prefill(wl, args, sets: int) -> dict:
    """One prefill chunk (compressor over the chunk, indexer + top-k and attention for its Q
    queries) per step: tokens/s, the fraction of the bf16 MFMA peak per op and for the step, and
    per-step percentiles."""
    R = max(1, min(sets, args.steps))
    log(f"[bench] {wl.name}: building {R} input sets")
    bench = Bench(wl, R, seed=1000)
    full, rem = divmod(args.steps, R)

    def timed(op):
        gs = [bench.graph(op)] * full + ([bench.graph(op, range(rem))] if rem else [])
        for _ in range(max(1, args.warmup // R)):
            gs[0].replay()
        return bench.time_steps(gs, 1, 0) / args.steps

    ms = {op: timed(op) for op in ["step", "compress", "index_topk", "attention"]}
    dist = bench.distribution("step")
    del bench
    import torch
    torch.cuda.empty_cache()
    fl = prefill_flops(wl)
    tflops = {k: fl[k] / (ms[k] * 1e-3) / 1e12 for k in ["index_topk", "attention", "step"]}
    for k in ms:
        log(f"[bench] {wl.name} {k}: {ms[k] * 1e3:.1f} us" + (f", {tflops[k]:.0f} TFLOP/s" if k in tflops else ""))
    dom = max(["index_topk", "attention"], key=lambda k: ms[k])
    roof = {op: {"bound": "mfma", "achieved": tflops[op], "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops[op] / BF16_MFMA_PEAK_TFLOPS, "traffic": measured_traffic(wl.name, op),
                 "flops_per_launch": fl[op],
                 "us_per_launch": ms[op] * 1e3,
                 "kernel": ("hcs_sparse_mla_prefill_chunk (mla_heads_kernel<512, head pairs>)" if op == "attention"
                            else "hcs_index_topk_chunk (index_score_chunk_kernel + topk_single_kernel)")}
            for op in ["index_topk", "attention"]}
    return {
        "metric": "prefill tokens/s and % bf16 MFMA peak, CSA chunk, 1 GPU", "value": wl.Q / (ms["step"] * 1e-3),
        "unit": "tokens/s", "ms_per_step": ms["step"], "timing": dist, "dtype": "bf16",
        "config": {"workload": wl.name, "P0": wl.P0, "Q": wl.Q, "heads": wl.H, "head_dim": wl.d,
                   "compress_ratio": wl.m, "window": wl.window, "topk": wl.topk,
                   "indexer": f"{wl.H_I}x{wl.d_I} bf16", "input_sets_rotated": R},
        "mfma_frac_step": tflops["step"] / BF16_MFMA_PEAK_TFLOPS, "flops_per_step": fl["step"],
        "roofline": roof[dom], "rooflines": roof,
        "ops_us": {k: v * 1e3 for k, v in ms.items()},
    }


# ------------------------------------------------------------------ decode workloads

def attention_kernel_name(wl, fused: bool) -> str:
    # the split merge is mla_combine_wave_kernel<512, 4> for at most four splits per query,
    # mla_combine_kernel<512> above that
    merge = "split merge"
    if fused:
        return f"hcs_sparse_mla_decode_select (mla_heads_kernel<512, select> + {merge})"
    if wl.kv_fmt == "bf16":
        return f"hcs_sparse_mla_decode (mla_heads_kernel<512> + {merge})"
    return f"hcs_sparse_mla_decode (mla_heads_kernel<512, quantized rows> + {merge})"


def index_kernel_name(wl, fused: bool) -> str:
    if fused:
        return "hcs_index_scores_compress (index_score_compress_kernel)"
    if wl.ix_fmt == "mxfp4":
        return "hcs_index_topk (index_score_mxfp4_kernel + topk_filter_kernel + topk_select_kernel)"
    return "hcs_index_topk (index_score_bf16_kernel + topk_single_kernel)"


def measure_decode(wl, args, sets: int, seed: int = 1000, two_call: bool = False) -> dict:
    """One decode workload: the step time over exactly args.steps steps (rotating `sets` input
    sets), per-step percentiles, each op's time and, for each HBM-bound op, its roofline entry
    (algorithmic bytes per launch / measured time per launch against the 8 TB/s peak)."""
    import torch

    n_vis = wl.ctx // wl.m
    R = max(1, min(sets, args.steps))
    log(f"[bench] {wl.name}: building {R} input sets")
    fused = select_in_attention_ok(wl) and not two_call
    bench = Bench(wl, R, seed=seed, select_in_attention=fused)

    def timed(op, steps, warmup):
        """ms per launch of `op` over exactly `steps` launches (after `warmup` untimed ones),
        rotating the input sets: full rounds of all sets, then the remainder."""
        full, rem = divmod(steps, R)
        gs = ([bench.graph(op)] * full) + ([bench.graph(op, range(rem))] if rem else [])
        wf, wr = divmod(warmup, R)
        for _ in range(wf):
            gs[0].replay()
        if wr:
            bench.graph(op, range(wr)).replay()
        return bench.time_steps(gs, 1, 0) / steps

    log(f"[bench] {wl.name}: capturing the step graph")
    ms_step = timed("step", args.steps, args.warmup)
    dist = bench.distribution("step")
    ops = ["compress", "attention"] + (["index_topk"] if wl.indexer else [])
    # with the selection inside the attention, the indexer op produces the scores only
    label = {"index_topk": "index_scores", "attention": "attention_select"} if fused else {}
    op_ms = {}
    for op in ops:
        op_ms[op] = timed(op, args.steps, args.warmup)
        log(f"[bench] {wl.name} {label.get(op, op)}: {op_ms[op] * 1e3:.2f} us")
    del bench
    torch.cuda.empty_cache()
    by = algo_bytes(wl, n_vis)
    qps = wl.B / (ms_step * 1e-3)
    step_gbs = by["step"] / (ms_step * 1e-3) / 1e9
    log(f"[bench] {wl.name}: step {ms_step * 1e3:.2f} us (p50 {dist['p50_ms'] * 1e3:.2f}), {qps:,.0f} q/s, "
        f"{step_gbs:.0f} GB/s ({100 * step_gbs / HBM_PEAK_GBS:.1f}% of HBM)")
    op_bytes = {"attention": by["attention"], "index_topk": by["index_topk"]}
    if fused:
        # the attention launch reads every visible entry's score instead of the selected ids,
        # and the indexer launch writes the scores instead of the ids
        op_bytes["attention"] += wl.B * (n_vis * 4 - min(wl.topk, n_vis) * 4)
        op_bytes["index_topk"] += wl.B * (n_vis * 4 - wl.topk * 8)
    roofs = {}
    for op in [o for o in ("attention", "index_topk") if o in op_ms]:
        gbs = op_bytes[op] / (op_ms[op] * 1e-3) / 1e9
        roofs[op] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name, op),
                     "kernel": attention_kernel_name(wl, fused) if op == "attention" else index_kernel_name(wl, fused),
                     "algorithmic_bytes_per_launch": op_bytes[op], "us_per_launch": op_ms[op] * 1e3}
    dom = max(roofs, key=lambda o: op_ms[o])
    return {
        "value": qps, "unit": "queries/s", "ms_per_step": ms_step, "timing": dist,
        "dtype": "bf16" if wl.kv_fmt == "bf16" else f"{wl.kv_fmt} KV + {wl.ix_fmt} indexer (bf16 / fp4 MFMA)",
        "config": {"workload": wl.name, "batch": wl.B, "context": wl.ctx, "heads": wl.H,
                   "head_dim": wl.d, "compress_ratio": wl.m, "window": wl.window,
                   "topk": wl.topk if wl.indexer else None,
                   "indexer": f"{wl.H_I}x{wl.d_I} {wl.ix_fmt}" if wl.indexer else None,
                   "kv_format": wl.kv_fmt, "input_sets_rotated": R},
        "hbm_tb_s": step_gbs / 1e3, "hbm_frac": step_gbs / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": by["step"],
        "roofline": roofs[dom], "rooflines": roofs,
        "ops_us": {label.get(k, k): v * 1e3 for k, v in op_ms.items()},
        "select_in_attention": fused,
    }


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="csa_decode_bf16")
    ap.add_argument("--sets", type=int, default=24,
                    help="independent input sets rotated per replay (the CSA decode workload's caches: "
                         "88 MB per set; fewer for the larger workloads)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure only --workload (no other workloads, no side measurements)")
    ap.add_argument("--two-call", action="store_true",
                    help="CSA decode: top-k in the indexer launch (hcs_index_topk_compress + "
                         "hcs_sparse_mla_decode) instead of inside the attention")
    ap.add_argument("--only", default=None, help="replay only this op's graph (for profiling)")
    ap.add_argument("--side", default=None, choices=["compress_full", "insert_decode", "insert_prefill",
                                                     "indexer_formats"],
                    help="run only this side measurement of the decode workload (for profiling)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="instead of the path: copy MIB MiB device to device --steps times (the known-size "
                         "reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only: the decode path of one "
                                   "layer needs no collectives; run with --gpus 1"}))
        sys.exit(2)

    import torch

    from synth import configs as C

    if args.calib_copy:
        n = args.calib_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n, "launches": args.steps}))
        return

    wl = C.BY_NAME[args.workload]
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")
    if args.side:
        if wl.kind != "decode":
            sys.exit("side measurements use a decode workload's shapes")
        R = max(1, min(args.sets, args.steps, 8))
        reps = max(1, args.steps // R)
        if args.side == "compress_full":
            res = bench_compress_full(wl, R, reps)
        elif args.side == "indexer_formats":
            res = bench_indexer_formats(wl, 16 if wl.ctx <= 65536 else 1, reps)
            res["us_per_call"] = res["mxfp4"]["us_per_call"]
        elif args.side == "insert_decode":
            res = bench_insert(wl, wl.B, 1, R, reps)
        else:
            res = bench_insert(wl, 1, 4096, R, reps)
        log(f"[bench] {args.side}: {res['us_per_call']:.2f} us")
        print(json.dumps({"side": args.side, **res}))
        return
    # input sets per workload: enough rotation that the 256 MB Infinity Cache cannot hold the
    # step's caches between uses (CSA decode: 88 MB per set; HCA: 72 MB; 1M: 1.36 GB; prefill:
    # 0.3 GB of q alone)
    sets_of = {"csa_decode_bf16": args.sets, "hca_decode_bf16": min(args.sets, 16),
               "csa_decode_1m_fp8": 2, "csa_decode_1m_v41": 2, "csa_prefill_bf16": 2}
    if wl.kind == "prefill":
        res = measure_prefill(wl, args, sets_of.get(wl.name, 2))
        print(json.dumps({"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "data": "synthetic", **res}))
        return
    if wl.kind != "decode":
        sys.exit("bench workloads are the decode and prefill configurations")

    if args.only:
        R = max(1, min(sets_of.get(wl.name, args.sets), args.steps))
        fused = select_in_attention_ok(wl) and not args.two_call
        bench = Bench(wl, R, seed=1000, select_in_attention=fused)
        if args.only != "step":
            # one round of whole steps first, so that the attention entry point reads rows
            # of a real selection (the top-k output it consumes)
            bench.graph("step").replay()
        full, rem = divmod(args.steps, R)
        gs = ([bench.graph(args.only)] * full) + ([bench.graph(args.only, range(rem))] if rem else [])
        ms = bench.time_steps(gs, 1, 0) / args.steps
        log(f"[bench] {args.only}: {ms * 1e3:.2f} us per launch")
        print(json.dumps({"op": args.only, "us_per_launch": ms * 1e3, "launches": args.steps}))
        return

    head = measure_decode(wl, args, sets_of.get(wl.name, args.sets), two_call=args.two_call)
    result = {"metric": METRIC, "value": head["value"], "unit": "queries/s", "n_gpus": 1,
              "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
              "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "data": "synthetic",
              **{k: v for k, v in head.items() if k not in ("value", "unit", "ms_per_step")}}

    if not args.no_extra and wl.name == "csa_decode_bf16":
        for other in (C.HCA_DECODE, C.CSA_DECODE_1M_FP8):
            res = measure_decode(other, args, sets_of[other.name], seed=2000)
            result[other.name] = res
        result[C.CSA_PREFILL.name] = measure_prefill(C.CSA_PREFILL, args, sets_of[C.CSA_PREFILL.name])
        R = max(1, min(args.sets, args.steps, 8))
        reps = max(1, args.steps // R)
        log("[bench] side measurement: full compressor at this decode step")
        result["compress_full"] = bench_compress_full(wl, R, reps)
        log(f"[bench] compress_full: {result['compress_full']['us_per_call']:.2f} us")
        log("[bench] side measurement: query preparation and SWA insert (decode step, prefill chunk)")
        result["qnorm_rope_kv_insert"] = {"decode": bench_insert(wl, wl.B, 1, R, reps),
                                          "prefill_chunk": bench_insert(wl, 1, 4096, R, reps)}
        for k, v in result["qnorm_rope_kv_insert"].items():
            log(f"[bench] qnorm_rope_kv_insert {k}: {v['us_per_call']:.2f} us, {v['gb_s']:.0f} GB/s "
                f"({100 * v['hbm_frac']:.1f}% of HBM)")
        log("[bench] side measurement: indexer key formats (bf16 / MXFP4 / FP8), time and recall")
        result["indexer_formats"] = {wl.name: bench_indexer_formats(wl, 16, max(1, reps // 2)),
                                     C.CSA_DECODE_1M_FP8.name: bench_indexer_formats(C.CSA_DECODE_1M_FP8, 1, reps)}
        for name, v in result["indexer_formats"].items():
            log(f"[bench] indexer {name}: " + ", ".join(
                f"{f} {v[f]['us_per_call']:.1f} us" + (f" (recall {100 * v[f]['recall_vs_bf16']:.2f}%)" if f != "bf16" else "")
                for f in ("bf16", "mxfp4", "fp8ix")))

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
