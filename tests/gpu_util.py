"""Helpers of the GPU parity tests: run a ``synth`` scenario through the HIP path and compare
its outputs with the oracle's.

Tolerances (from the arithmetic of the kernels):
  * compressed entries, float32 copy: per entry max_c |gpu - ref| <= 1e-3 * max_c |ref|
    (float32 online softmax vs float64);
  * stored bf16 entries: within one bf16 ulp of the oracle's float64 entry rounded to bf16;
  * top-k: the id sets agree except ids whose oracle score is within 1e-4 (relative) of the
    oracle's k-th score (near-ties may go either way);
  * attention output: max |gpu - ref| <= 2e-2 (bf16 KV) / 6e-2 (fp8 KV), and the relative
    Frobenius error <= 1e-2: q and the rows are exact bf16 inputs, the logits and the output
    accumulate in float32, the probabilities enter the PV product as bf16 (relative 2^-9) and
    the output is rounded to bf16 (relative 2^-9).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import hybrid_compressed_sparse_amd as hcs
from hybrid_compressed_sparse_amd.step import PathStep, StepShape
from oracle import formats as OF
from oracle import pipeline as OP

ATTN_TOL = {"bf16": 2e-2, "fp8ds": 6e-2, "mxfp8": 6e-2}
REL_FRO = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def shape_of(sc) -> StepShape:
    wl = sc.wl
    return StepShape(N=sc.N, H=wl.H, d=wl.d, m=wl.m, window=wl.window, max_pos=sc.max_pos(),
                     topk=wl.topk if wl.indexer else 0, prefill=wl.kind == "prefill",
                     seq=0, P0=wl.P0)


def _ix_q_args(sc):
    if isinstance(sc.ix_q, torch.Tensor):
        return sc.ix_q.contiguous(), None
    return sc.ix_q.codes.contiguous(), sc.ix_q.scales.contiguous()


def compress_calls(sc, state, comp_override=None, dbg=None, split_at=None):
    """Run the compressor over each sequence's stream: the setup tokens (all but the step's own)
    in one call, then the step's tokens. split_at: extra cut points (tokens from the stream start)
    that split the setup into more calls, to exercise the state carried between calls.
    Returns the start position of each sequence's last call (its entries go to ``dbg``)."""
    dev = sc.c_x.device
    B = len(sc.c_cu) - 1
    lens = [sc.c_cu[b + 1] - sc.c_cu[b] for b in range(B)]
    starts = sc.c_start.tolist()
    bounds = []
    for b in range(B):
        step_lo = max(0, lens[b] - sc.n_step)
        cb = sorted(set([0, step_lo, lens[b]] + [c for c in (split_at or []) if 0 < c < step_lo]))
        bounds.append(cb)
    ncalls = max(len(cb) - 1 for cb in bounds)
    comp = comp_override if comp_override is not None else sc.comp
    last_start = [0] * B
    for k in range(ncalls):
        rows, cu, st = [], [0], []
        max_new = 1
        for b in range(B):
            cb = bounds[b]
            # sequences with fewer cuts take their last calls at the end
            j = k - (ncalls - (len(cb) - 1))
            lo, hi = (cb[j], cb[j + 1]) if j >= 0 else (0, 0)
            rows.append(torch.arange(sc.c_cu[b] + lo, sc.c_cu[b] + hi, device=dev))
            cu.append(cu[-1] + (hi - lo))
            st.append(starts[b] + lo)
            if k == ncalls - 1:
                last_start[b] = starts[b] + lo
            max_new = max(max_new, hi - lo)
        r = torch.cat(rows)
        kv = sc.c_x.index_select(0, r).contiguous()
        sc_ = sc.c_s.index_select(0, r).contiguous()
        hcs.compress_kv(kv, sc_, torch.tensor(cu, dtype=torch.int32, device=dev),
                        torch.tensor(st, dtype=torch.int32, device=dev), state, comp, sc.wl.m,
                        ape=sc.ape, dbg=dbg if k == ncalls - 1 else None, max_new=max_new)
    return last_start


def run_step(sc, topk_override=None, sink=None, split_at=None, dbg_rows=None):
    """The whole step on the GPU. Returns (PathStep, dbg float32 copy of the step's entries)."""
    wl = sc.wl
    dev = sc.c_x.device
    B = len(sc.c_cu) - 1
    step = PathStep(shape_of(sc), device=dev)
    state = torch.zeros((B, 3 * wl.d), dtype=torch.float32, device=dev)
    rows = dbg_rows if dbg_rows is not None else sc.n_step // wl.m + 2
    dbg = torch.full((B, rows, wl.d), float("nan"), dtype=torch.float32, device=dev)
    step.last_start = compress_calls(sc, state, dbg=dbg, split_at=split_at)
    if wl.indexer and topk_override is None:
        q, qs = _ix_q_args(sc)
        step.select(q, qs, sc.ix_w.contiguous(), sc.ix, sc.q_seq, sc.q_pos)
    step.attend(sc.q, sc.swa, sc.comp, sc.q_seq, sc.q_pos, sink=sink, topk_idx=topk_override)
    torch.cuda.synchronize()
    return step, dbg


# ------------------------------------------------------------------ comparisons

def check_entries(sc, step, dbg, produced, b: int):
    """GPU float32 entry copy and stored cache rows of sequence b vs the oracle."""
    first, C, _ = produced[b]
    n = C.shape[0]
    if n == 0:
        return
    m = sc.wl.m
    first_dbg = step.last_start[b] // m       # dbg row 0 = first block touched by the last call
    got = dbg[b].double().cpu().numpy()
    i0 = max(first, first_dbg)
    if i0 < first + n:
        g = got[i0 - first_dbg: first + n - first_dbg]
        r = C[i0 - first:]
        err = np.abs(g - r).max(axis=1)
        lim = 1e-3 * np.abs(r).max(axis=1)
        assert np.all(err <= lim), f"entry error {err.max()} (limit {lim.min()})"
    # stored rows in the cache
    from synth import layout as L
    ids = torch.arange(first, first + n, device=sc.comp.pool.device)
    fmt = sc.wl.cfmt
    stored = L.gather_rows(sc.comp.pool, fmt, sc.wl.d, sc.comp.page_table[b], ids)
    if fmt in ("mxfp8", "nvfp4"):
        check_v41_rows(fmt, stored, C)
        return
    if fmt == "bf16":
        # the stored value is the GPU's float32 entry rounded to nearest bf16: within half a bf16
        # ulp of it, and the float32 entry is within 1e-4 of the row's scale of the exact one
        gv = OF.decode_bf16(stored.view(torch.int16).cpu().numpy().view(np.uint16))
        _, e = np.frexp(np.abs(gv))
        half_ulp = np.ldexp(1.0, e - 1 - 8)
        lim = half_ulp + 1e-4 * np.abs(C).max(axis=1, keepdims=True)
        assert np.all(np.abs(gv - C) <= lim), "stored bf16 entry is not the rounded entry"
    else:
        gv = OP.decode_rows("fp8ds", stored)
        rec = OF.quantize_fp8ds(C.astype(np.float32))
        rv = OF.decode_fp8ds(*rec)
        same_codes = (stored.codes.cpu().numpy() == rec[0]).mean()
        assert same_codes >= 0.999, f"only {same_codes:.4f} of e4m3 codes agree"
        # a differing code is a rounding-boundary case: at most one e4m3 step (<= 32 * scale)
        step_ = np.repeat(OF.decode_ue8m0(rec[2]), 64, axis=-1) * 32.0
        assert np.all(np.abs(gv[:, :448] - rv[:, :448]) <= step_)
        assert np.all(np.abs(gv[:, 448:] - rv[:, 448:]) <= np.abs(rv[:, 448:]) * 2.0 ** -7 + 1e-30)


def _nibbles(packed: np.ndarray) -> np.ndarray:
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def check_v41_rows(fmt: str, stored, C: np.ndarray, min_same: float = 0.999):
    """Stored MXFP8 / NVFP4 rows against the oracle's encoding of the float64 rows C: codes and
    scales agree at least min_same (both sides decide them on float32 values computed in
    different orders), and every decoded value is within one step of the oracle's."""
    codes = stored.codes.cpu().numpy()
    scales = stored.scales.cpu().numpy()
    gv = OP.decode_rows(fmt, stored)
    if fmt == "mxfp8":
        rc, rs = OF.quantize_mxfp8(C.astype(np.float32))
        rv = OF.decode_mxfp8(rc, rs)
        assert (codes == rc).mean() >= min_same, f"only {(codes == rc).mean():.4f} of e4m3 codes agree"
        assert (scales == rs).mean() >= min_same
        step_ = np.repeat(OF.decode_ue8m0(rs), 32, axis=-1) * 32.0
        assert np.all(np.abs(gv - rv) <= step_)
    else:
        rc, rs = OF.quantize_nvfp4(C.astype(np.float32))
        rv = OF.decode_nvfp4(rc, rs)
        same = (_nibbles(codes) == _nibbles(rc)).mean()
        assert same >= min_same, f"only {same:.4f} of e2m1 codes agree"
        assert (scales == rs).mean() >= min_same
        # one e2m1 step (at most 2) of the larger of the two scales
        sv = np.maximum(OF.decode_e4m3(rs), OF.decode_e4m3(scales))
        assert np.all(np.abs(gv - rv) <= np.repeat(sv, 16, axis=-1) * 2.0 + 1e-30)


def check_topk(gpu_idx: np.ndarray, gpu_score: np.ndarray, ref_idx: np.ndarray, ref_scores: np.ndarray,
               k: int):
    """Set comparison with the near-tie rule; GPU scores of its own ids vs the oracle's."""
    nv = ref_scores.shape[0]
    G = set(int(i) for i in gpu_idx if i >= 0)
    O = set(int(i) for i in ref_idx if i >= 0)
    assert len(G) == min(k, nv), f"gpu selected {len(G)} distinct ids, expected {min(k, nv)}"
    assert all(0 <= i < nv for i in G)
    assert int((gpu_idx >= 0).sum()) == min(k, nv)
    if nv <= k:
        assert G == O
        return
    sk = ref_scores[int(ref_idx[k - 1])]
    for i in G ^ O:
        assert abs(ref_scores[i] - sk) <= 1e-4 * abs(sk) + 1e-30, \
            f"id {i} score {ref_scores[i]} not a near-tie of k-th {sk}"
    sel = gpu_idx >= 0
    err = np.abs(gpu_score[sel] - ref_scores[gpu_idx[sel]])
    assert err.max() <= 1e-4 * abs(sk) + 1e-6, f"score error {err.max()}"


def check_attention(o_gpu: np.ndarray, o_ref: np.ndarray, fmt: str, lse_gpu=None, lse_ref=None):
    err = np.abs(o_gpu - o_ref).max()
    fro = np.linalg.norm(o_gpu - o_ref) / max(np.linalg.norm(o_ref), 1e-30)
    assert err <= ATTN_TOL[fmt], f"max abs error {err}"
    assert fro <= REL_FRO, f"relative Frobenius error {fro}"
    if lse_gpu is not None:
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse_gpu))
        assert np.abs(lse_gpu[fin] - lse_ref[fin]).max() <= 1e-3
    return err, fro


def out_np(step, t):
    return step.out[t].float().cpu().numpy().astype(np.float64)
