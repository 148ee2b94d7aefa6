"""Pins of the oracle's whole step on seeded scenarios, and the pages' printed numbers (CPU only)."""
import os

import numpy as np
import torch

from oracle import method as M
from oracle import pipeline as P
from synth import configs as C
from synth import gen as G
from synth import layout as L


def _golden(golden_dir, name):
    out = {}
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                k, *v = line.split()
                out[k] = v
    return out


def test_concrete_trace_numbers(golden_dir):
    g = _golden(golden_dir, "concrete_trace.txt")
    p, m = int(g["position"][0]), int(g["compress_ratio"][0])
    assert M.n_visible(p, m) == int(g["compressed_available"][0])
    swa, comp = M.row_set(p, int(g["window"][0]), m, np.arange(int(g["topk"][0])))
    assert swa.size + comp.size == int(g["attended_total"][0])
    assert abs(p / (swa.size + comp.size) - int(g["reduction_approx"][0])) < 1.5


def test_record_widths(golden_dir):
    g = _golden(golden_dir, "record_widths.txt")
    assert L.row_bytes(L.FMT_FP8DS, int(g["fp8ds"][0])) == int(g["fp8ds"][1])
    assert L.row_bytes(L.FMT_MXFP4, int(g["mxfp4"][0])) == int(g["mxfp4"][1])


def _sdpa_masked(q, rows, scale, mask):
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(rows)[None, None].expand(1, q.shape[0], -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, kt, attn_mask=torch.from_numpy(mask)[None, None, None, :], scale=scale)
    return out[0, :, 0, :].numpy()


def test_tiny_step_equals_dense_masked_attention():
    sc = G.build(C.TINY_CSA, seed=0)
    res = P.step(sc)
    first, Cf, stored = res["produced"][0]
    assert first == 0 and Cf.shape == (256, 128)
    X = P.decode_input(sc.c_x)                       # the raw rows double as the window rows
    for t in range(sc.N):
        p = int(sc.q_pos[t])
        nv = M.n_visible(p, 4)
        scores = res["scores"][t]
        assert scores.shape == (nv,)
        assert np.array_equal(res["topk"][t], np.argsort(-scores, kind="stable")[:32])
        allrows = np.concatenate([X, stored])
        mask = np.zeros(allrows.shape[0], dtype=bool)
        mask[max(0, p - 15): p + 1] = True
        mask[X.shape[0] + res["topk"][t]] = True
        q = P.decode_rows("bf16", sc.q[t])
        ref = _sdpa_masked(q, allrows, 128 ** -0.5, mask)
        assert np.allclose(res["o"][t], ref, atol=1e-12)


def test_step_hca_ratio_one_no_window_is_causal_attention():
    wl = C.Workload(name="hca_m1", kind="tiny", B=1, ctx=64, H=4, d=32, d_rope=8, m=1, window=0,
                    indexer=False, in_dtype="bf16", n_query=8, q_std=1.0)
    sc = G.build(wl, seed=3)
    res = P.step(sc)
    X = P.decode_input(sc.c_x)
    Q = np.stack([P.decode_rows("bf16", sc.q[t]) for t in range(sc.N)])      # [8, H, d]
    qt = torch.from_numpy(Q).permute(1, 0, 2)[None]                          # [1, H, 8, d]
    kt = torch.from_numpy(X)[None, None].expand(1, 4, 64, 32)
    mask = torch.from_numpy(np.arange(64)[None, :] <= np.arange(56, 64)[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, attn_mask=mask, scale=32 ** -0.5)
    ref = ref[0].permute(1, 0, 2).numpy()
    for t in range(sc.N):
        assert np.allclose(res["o"][t], ref[t], atol=1e-12)


def test_step_reads_back_what_it_stored_fp8ds():
    """The produced entry of an fp8_ds step is the oracle's own quantized record."""
    wl = C.CSA_DECODE_1M_FP8.with_(B=2, ctx=4096, topk=64)
    sc = G.build(wl, seed=1)
    res = P.step(sc, queries=[0])
    first, Cf, stored = res["produced"][0]
    assert first == 1023 and Cf.shape == (1, 512)
    lat = np.abs(stored[0, :448] - Cf[0, :448])
    assert lat.max() <= np.abs(Cf[0, :448]).max() / 16          # within e4m3 resolution
    vals = P.comp_values(sc, 0, np.array([first, 5]), res["produced"])
    assert np.array_equal(vals[0], stored[0])
