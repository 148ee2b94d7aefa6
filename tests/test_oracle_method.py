"""Pins of the oracle's method: closed forms, invariants and library routines (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import method as M



# ------------------------------------------------------------------ compressor

def test_compressor_weights_sum_to_one_per_channel():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((64, 16))
    S = rng.standard_normal((64, 16)) * 5
    C, alpha = M.compress(X, S, 4)
    assert alpha.shape == (16, 4, 16)
    assert np.allclose(alpha.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(alpha > 0)
    # a constant row stream compresses to the same constant
    C1, _ = M.compress(np.full((64, 16), 0.3), S, 4)
    assert np.allclose(C1, 0.3, atol=1e-15)


def test_compressor_ratio_one_is_identity():
    rng = np.random.default_rng(1)
    X = rng.standard_normal((37, 8))
    C, _ = M.compress(X, rng.standard_normal((37, 8)), 1)
    assert np.array_equal(C, X)


def test_compressor_equal_logits_give_the_mean():
    rng = np.random.default_rng(2)
    X = rng.standard_normal((128 * 3, 8))
    S = np.repeat(rng.standard_normal((3, 1, 8)), 128, axis=1).reshape(384, 8)
    C, _ = M.compress(X, S, 128)
    assert np.allclose(C, X.reshape(3, 128, 8).mean(axis=1), atol=1e-14)


def test_compressor_dominant_logit_selects_its_row():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((8, 4))
    S = rng.standard_normal((8, 4))
    S[2, :] += 1000.0      # token 2 of block 0
    S[7, 1] += 1000.0      # token 3 of block 1, channel 1 only
    C, _ = M.compress(X, S, 4)
    assert np.allclose(C[0], X[2])
    assert np.isclose(C[1, 1], X[7, 1])


def test_compressor_closed_form_two_tokens():
    # logits 0 and ln 3 -> weights 1/4, 3/4
    X = np.array([[1.0, -2.0], [5.0, 2.0]])
    S = np.array([[0.0, math.log(3.0)], [math.log(3.0), 0.0]])
    C, _ = M.compress(X, S, 2)
    assert np.allclose(C[0], [0.25 * 1 + 0.75 * 5, 0.75 * -2 + 0.25 * 2])


def test_compressor_ape_shifts_logits_per_block_position():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((16, 6))
    S = rng.standard_normal((16, 6))
    # an encoding constant across block positions cancels in the softmax
    C0, _ = M.compress(X, S, 4)
    Cc, _ = M.compress(X, S, 4, ape=np.tile(rng.standard_normal((1, 6)), (4, 1)))
    assert np.allclose(C0, Cc)
    # a dominant encoding at position 1 picks token 1 of every block
    ape = np.zeros((4, 6))
    ape[1] = 1000.0
    C1, _ = M.compress(X, S, 4, ape=ape)
    assert np.allclose(C1, X.reshape(4, 4, 6)[:, 1])


def test_compressor_partial_block_makes_no_entry():
    C, _ = M.compress(np.ones((7, 3)), np.zeros((7, 3)), 4)
    assert C.shape == (1, 3)
    C, _ = M.compress(np.ones((3, 3)), np.zeros((3, 3)), 4)
    assert C.shape == (0, 3)


def test_visibility_counts():
    assert M.n_visible(8191, 4) == 2048
    assert M.n_visible(131071, 128) == 1024
    assert M.n_visible(1048575, 4) == 262144
    assert M.n_visible(65536, 4) == 16384 and M.n_visible(69631, 4) == 17408
    assert M.n_visible(2, 4) == 0 and M.n_visible(3, 4) == 1


# ------------------------------------------------------------------ indexer / top-k

def test_index_single_head_is_relu_dot():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 32))
    K = rng.standard_normal((100, 32))
    s = M.index_scores(q, np.ones(1), K)
    assert np.allclose(s, np.maximum(np.dot(K, q[0]), 0.0))
    assert np.all(s[np.dot(K, q[0]) < 0] == 0.0)


def test_index_linear_in_weights_and_sum_over_heads():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((4, 16))
    K = rng.standard_normal((50, 16))
    w1, w2 = rng.uniform(size=4), rng.uniform(size=4)
    assert np.allclose(M.index_scores(q, w1 + w2, K), M.index_scores(q, w1, K) + M.index_scores(q, w2, K))
    per_head = sum(w1[h] * np.maximum(K @ q[h], 0) for h in range(4))
    assert np.allclose(M.index_scores(q, w1, K), per_head)


def test_topk_matches_library_stable_sort():
    rng = np.random.default_rng(7)
    s = rng.standard_normal(1000)
    s[::7] = 0.5          # many exact ties
    ids = M.topk(s, 100)
    lib = np.argsort(-s, kind="stable")[:100]
    assert np.array_equal(ids, lib)
    # ties resolved towards the smaller index
    tie = M.topk(np.array([1.0, 2.0, 2.0, 2.0, 0.0]), 2)
    assert tie.tolist() == [1, 2]


def test_topk_short_context_selects_all_and_pads():
    s = np.array([0.1, 0.9, 0.3])
    ids = M.topk(s, 5)
    assert ids.tolist() == [1, 2, 0, -1, -1]
    assert M.topk(np.zeros(0), 4).tolist() == [-1, -1, -1, -1]


# ------------------------------------------------------------------ attention

def _sdpa(q, rows, scale, mask=None):
    """torch's scaled_dot_product_attention in float64 (library routine), one KV head."""
    qt = torch.from_numpy(q)[None, :, None, :]                         # [1, H, 1, d]
    kt = torch.from_numpy(rows)[None, None].expand(1, q.shape[0], -1, -1)  # [1, H, R, d]
    out = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, kt,
        attn_mask=None if mask is None else torch.from_numpy(mask)[None, None, None, :],
        scale=scale)
    return out[0, :, 0, :].numpy()


def test_attention_matches_sdpa_and_logsumexp():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((8, 64)) * 3
    rows = rng.standard_normal((40, 64))
    o, lse = M.attention(q, rows, 0.125)
    assert np.allclose(o, _sdpa(q, rows, 0.125), atol=1e-12)
    ref_lse = torch.logsumexp(torch.from_numpy(0.125 * q @ rows.T), dim=1).numpy()
    assert np.allclose(lse, ref_lse, atol=1e-12)


def test_attention_sink_forms():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((4, 16))
    rows = rng.standard_normal((10, 16))
    o, lse = M.attention(q, rows, 0.25)
    o_inf, lse_inf = M.attention(q, rows, 0.25, sink=np.full(4, -np.inf))
    assert np.allclose(o, o_inf) and np.allclose(lse, lse_inf)
    sink = np.array([0.0, 1.0, -2.0, 5.0])
    o_s, lse_s = M.attention(q, rows, 0.25, sink=sink)
    z = np.exp(lse)                                   # sum_r e^{l}
    assert np.allclose(o_s, o * (z / (z + np.exp(sink)))[:, None])
    assert np.allclose(lse_s, np.log(z + np.exp(sink)))


def test_attention_single_row_and_duplicates():
    rng = np.random.default_rng(10)
    q = rng.standard_normal((3, 8))
    r = rng.standard_normal((1, 8))
    o, _ = M.attention(q, r, 1.0)
    assert np.allclose(o, np.repeat(r, 3, axis=0))
    rows = rng.standard_normal((6, 8))
    # a row listed twice behaves as that row with its logit raised by ln 2
    o2, _ = M.attention(q, np.concatenate([rows, rows[:2]]), 0.5)
    logits = 0.5 * q @ rows.T
    logits[:, :2] += math.log(2.0)
    p = np.exp(logits - logits.max(1, keepdims=True))
    assert np.allclose(o2, (p @ rows) / p.sum(1, keepdims=True))


def test_attention_empty_row_set():
    o, lse = M.attention(np.ones((2, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


def test_sparse_rows_equal_dense_attention_with_mask():
    """Sparse selection == dense attention over every row with a mask (library SDPA)."""
    rng = np.random.default_rng(11)
    m, w, p, H, d = 4, 16, 1022, 8, 32
    raw = rng.standard_normal((p + 1, d))
    comp = rng.standard_normal((M.n_visible(p, m), d))
    sel = rng.choice(comp.shape[0], 20, replace=False)
    sel = np.concatenate([sel, [-1, -1, comp.shape[0] + 5]])     # padding / invisible ids are ignored
    q = rng.standard_normal((H, d))
    swa, cid = M.row_set(p, w, m, sel)
    o, _ = M.attention(q, np.concatenate([raw[swa], comp[cid]]), d ** -0.5)
    allrows = np.concatenate([raw, comp])
    mask = np.zeros(allrows.shape[0], dtype=bool)
    mask[swa] = True
    mask[raw.shape[0] + cid] = True
    assert np.allclose(o, _sdpa(q, allrows, d ** -0.5, mask), atol=1e-12)


def test_hca_ratio_one_no_window_is_full_causal_attention():
    """HCA with m=1, no window and no top-k: every earlier token is one compressed entry,
    so the path is full causal attention over the raw rows (torch SDPA, is_causal)."""
    rng = np.random.default_rng(12)
    T, H, d = 50, 4, 16
    X = rng.standard_normal((T, d))
    C, _ = M.compress(X, rng.standard_normal((T, d)), 1)
    Q = rng.standard_normal((T, H, d))
    outs = []
    for p in range(T):
        swa, cid = M.row_set(p, 0, 1, None)
        assert swa.size == 0 and cid.tolist() == list(range(p + 1))
        outs.append(M.attention(Q[p], C[cid], d ** -0.5)[0])
    ours = np.stack(outs)                                             # [T, H, d]
    qt = torch.from_numpy(Q).permute(1, 0, 2)[None]                   # [1, H, T, d]
    kt = torch.from_numpy(X)[None, None].expand(1, H, T, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, is_causal=True, scale=d ** -0.5)
    assert np.allclose(ours, ref[0].permute(1, 0, 2).numpy(), atol=1e-12)


def test_window_rows_include_own_token():
    swa, comp = M.row_set(500000, 128, 4, np.arange(1024))
    assert swa[0] == 500000 - 127 and swa[-1] == 500000 and swa.size == 128
    assert comp.size == 1024
    swa0, _ = M.row_set(5, 128, 4, None)
    assert swa0.tolist() == list(range(6))
