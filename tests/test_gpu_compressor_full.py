"""Parity of the full compressor (hcs_compress_kv_full: overlapping window, RMSNorm, RoPE) with
the oracle's compress_full, on seeded synthetic streams; state carried across calls."""
import math

import numpy as np
import pytest
import torch

import hybrid_compressed_sparse_amd as hcs
from oracle import formats as OF
from oracle import method as OM
from oracle import pipeline as OP
from synth import layout as L

pytestmark = pytest.mark.gpu


def _dev():
    return torch.device("cuda:0")


def _inputs(seed, lens, d, m, coff, with_ape, with_norm, d_rope):
    g = torch.Generator().manual_seed(seed)
    X = [(torch.randn(n, coff * d, generator=g) / math.sqrt(d)).to(torch.bfloat16) for n in lens]
    S = [torch.randn(n, coff * d, generator=g).to(torch.bfloat16) for n in lens]
    ape = torch.randn(m, coff * d, generator=g) * 0.5 if with_ape else None
    w = torch.rand(d, generator=g) * 1.5 + 0.25 if with_norm else None
    rows = m * max(1, max(lens) // m) + 1
    ang = torch.rand(rows, max(d_rope // 2, 1), generator=g, dtype=torch.float64) * 6.0 - 3.0
    cos = torch.cos(ang).float() if d_rope else None
    sin = torch.sin(ang).float() if d_rope else None
    return X, S, ape, w, cos, sin


def _cache(seed, lens, d, m, fmt, dev):
    n_ent = [n // m for n in lens]
    pages = [max(1, (e + 63) // 64) for e in n_ent]
    g = torch.Generator().manual_seed(seed + 99)
    perm = torch.randperm(sum(pages), generator=g).to(torch.int32)
    stride = max(pages)
    pt = torch.full((len(lens), stride), -1, dtype=torch.int32)
    k = 0
    for b, p in enumerate(pages):
        pt[b, :p] = perm[k: k + p]
        k += p
    pool = L.new_pool(sum(pages), fmt, d, dev)
    return pool, pt.to(dev)


def _run(X, S, ape, w, cos, sin, lens, d, m, coff, fmt, cuts, seed, eps=1e-6):
    """Run the compressor over each stream in calls cut at `cuts` (token offsets, per call the
    same cut for every stream, clipped to its length). Returns (pool, page_table, state, dbg of the
    last call, start positions of the last call)."""
    dev = _dev()
    B = len(lens)
    pool, pt = _cache(seed, lens, d, m, fmt, dev)
    comp = hcs.paged(pool, pt, fmt, d)
    state = torch.zeros((B, 3 * coff * d), dtype=torch.float32, device=dev)
    bounds = sorted(set([0] + [c for c in cuts if c > 0] + [max(lens)]))
    dbg = starts = None
    for k in range(len(bounds) - 1):
        lo, hi = bounds[k], bounds[k + 1]
        seg = [(min(lo, n), min(hi, n)) for n in lens]
        kv = torch.cat([X[b][a:e] for b, (a, e) in enumerate(seg)]).to(dev)
        sc = torch.cat([S[b][a:e] for b, (a, e) in enumerate(seg)]).to(dev)
        cu = torch.tensor([0] + list(np.cumsum([e - a for a, e in seg])), dtype=torch.int32, device=dev)
        st = torch.tensor([a for a, _ in seg], dtype=torch.int32, device=dev)
        last = k == len(bounds) - 2
        rows = (hi - lo) // m + 2
        dbg_k = torch.full((B, rows, d), float("nan"), dtype=torch.float32, device=dev) if last else None
        hcs.compress_kv_full(kv, sc, cu, st, state, comp, m, coff,
                             ape=None if ape is None else ape.to(dev),
                             norm_weight=None if w is None else w.to(dev), norm_eps=eps,
                             rope_cos=None if cos is None else cos.to(dev),
                             rope_sin=None if sin is None else sin.to(dev), dbg=dbg_k,
                             max_new=max(1, hi - lo))
        if last:
            dbg, starts = dbg_k, [a for a, _ in seg]
    torch.cuda.synchronize()
    return pool, pt, state, dbg, starts


def _oracle(X, S, ape, w, cos, sin, m, coff, d_rope, eps=1e-6):
    out = []
    for Xb, Sb in zip(X, S):
        x = OP.decode_input(Xb)
        s = OP.decode_input(Sb)
        out.append(OM.compress_full(x, s, m, coff, ape=None if ape is None else ape.double().numpy(),
                                    norm_weight=None if w is None else w.double().numpy(), eps=eps,
                                    cos_table=None if cos is None else cos.double().numpy(),
                                    sin_table=None if sin is None else sin.double().numpy(),
                                    d_rope=d_rope))
    return out


def _check(pool, pt, dbg, starts, ref, lens, d, m, fmt):
    for b, C in enumerate(ref):
        n = C.shape[0]
        if n == 0:
            continue
        # the float32 entries of the last call
        k0 = starts[b] // m
        k1 = lens[b] // m
        if k1 > k0:
            got = dbg[b, : k1 - k0].double().cpu().numpy()
            err = np.abs(got - C[k0:k1]).max(axis=1)
            assert np.all(err <= 1e-3 * np.abs(C[k0:k1]).max(axis=1)), (b, err.max())
        # every stored row
        ids = torch.arange(n, device=pool.device)
        stored = L.gather_rows(pool, fmt, d, pt[b], ids)
        if fmt == "bf16":
            gv = OF.decode_bf16(stored.view(torch.int16).cpu().numpy().view(np.uint16))
            _, e = np.frexp(np.abs(gv))
            lim = np.ldexp(1.0, e - 9) + 1e-4 * np.abs(C).max(axis=1, keepdims=True)
            assert np.all(np.abs(gv - C) <= lim), b
        else:
            gv = OP.decode_rows("fp8ds", stored)
            rec = OF.quantize_fp8ds(C.astype(np.float32))
            rv = OF.decode_fp8ds(*rec)
            assert (stored.codes.cpu().numpy() == rec[0]).mean() >= 0.999
            step_ = np.repeat(OF.decode_ue8m0(rec[2]), 64, axis=-1) * 32.0
            assert np.all(np.abs(gv[:, :448] - rv[:, :448]) <= step_)
            # rotary dims in bf16: one bf16 step of the oracle's value, plus the float32 entry's
            # own error (rotated values can cancel to near zero, so it is taken on the row's scale)
            lim = np.abs(rv[:, 448:]) * 2.0 ** -7 + 1e-4 * np.abs(C).max(axis=1, keepdims=True)
            assert np.all(np.abs(gv[:, 448:] - rv[:, 448:]) <= lim)


@pytest.mark.parametrize("cuts", [[], [13, 16, 50]], ids=["one_call", "calls_cut_mid_and_at_blocks"])
def test_full_compressor_overlap_small(cuts):
    lens, d, m, coff, dr = [70, 9, 133], 128, 4, 2, 32
    X, S, ape, w, cos, sin = _inputs(31, lens, d, m, coff, True, True, dr)
    pool, pt, state, dbg, starts = _run(X, S, ape, w, cos, sin, lens, d, m, coff, "bf16", cuts, 31)
    _check(pool, pt, dbg, starts, _oracle(X, S, ape, w, cos, sin, m, coff, dr), lens, d, m, "bf16")


def test_full_compressor_calls_split_anywhere_give_the_same_bits():
    lens, d, m, coff, dr = [70, 9, 133], 128, 4, 2, 32
    X, S, ape, w, cos, sin = _inputs(32, lens, d, m, coff, True, True, dr)
    a = _run(X, S, ape, w, cos, sin, lens, d, m, coff, "bf16", [], 32)
    b = _run(X, S, ape, w, cos, sin, lens, d, m, coff, "bf16", [1, 2, 3, 4, 8, 13, 16, 17, 50, 99], 32)
    assert torch.equal(a[0], b[0]) and torch.equal(a[2], b[2])


def test_full_compressor_decode_step_fp8ds():
    """CSA at config-2 widths: d 512, m 4, fp8_ds entries with 64 rotary dims; the step's token
    arrives in a call of its own after the prefix."""
    lens, d, m, coff, dr = [2049, 4097, 1, 777], 512, 4, 2, 64
    X, S, ape, w, cos, sin = _inputs(33, lens, d, m, coff, False, True, dr)
    pool, pt, state, dbg, starts = _run(X, S, ape, w, cos, sin, lens, d, m, coff, "fp8ds", [], 33)
    _check(pool, pt, dbg, starts, _oracle(X, S, ape, w, cos, sin, m, coff, dr), lens, d, m, "fp8ds")
    # calls ending one token before each stream's end (its decode step): the same bits
    pool2, _, state2, _, _ = _run(X, S, ape, w, cos, sin, lens, d, m, coff, "fp8ds",
                                  [n - 1 for n in lens if n > 1], 33)
    assert torch.equal(pool, pool2) and torch.equal(state, state2)


def test_full_compressor_hca_norm_rope_no_overlap():
    lens, d, m, coff, dr = [1025, 300], 512, 128, 1, 64
    X, S, ape, w, cos, sin = _inputs(34, lens, d, m, coff, True, True, dr)
    pool, pt, state, dbg, starts = _run(X, S, ape, w, cos, sin, lens, d, m, coff, "bf16", [640], 34)
    _check(pool, pt, dbg, starts, _oracle(X, S, ape, w, cos, sin, m, coff, dr), lens, d, m, "bf16")


def test_full_compressor_without_epilogue_is_the_plain_compressor():
    """coff 1, no norm, no RoPE: the same bits as hcs_compress_kv (cache and state)."""
    dev = _dev()
    lens, d, m = [70, 9, 133], 128, 4
    X, S, ape, _, _, _ = _inputs(35, lens, d, m, 1, True, False, 0)
    a = _run(X, S, ape, None, None, None, lens, d, m, 1, "bf16", [13, 50], 35)
    pool, pt = _cache(35, lens, d, m, "bf16", dev)
    state = torch.zeros((len(lens), 3 * d), dtype=torch.float32, device=dev)
    comp = hcs.paged(pool, pt, "bf16", d)
    for lo, hi in [(0, 13), (13, 50), (50, max(lens))]:
        seg = [(min(lo, n), min(hi, n)) for n in lens]
        kv = torch.cat([X[b][x:y] for b, (x, y) in enumerate(seg)]).to(dev)
        sc = torch.cat([S[b][x:y] for b, (x, y) in enumerate(seg)]).to(dev)
        cu = torch.tensor([0] + list(np.cumsum([y - x for x, y in seg])), dtype=torch.int32, device=dev)
        st = torch.tensor([x for x, _ in seg], dtype=torch.int32, device=dev)
        hcs.compress_kv(kv, sc, cu, st, state, comp, m, ape=ape.to(dev), max_new=hi - lo)
    torch.cuda.synchronize()
    assert torch.equal(a[0], pool)
