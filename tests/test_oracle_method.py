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


# ------------------------------------------------------------------ full compressor (coff 2, epilogue)

def test_overlap_weights_sum_to_one_and_entry0_has_no_overlap():
    rng = np.random.default_rng(20)
    X = rng.standard_normal((40, 12))
    S = rng.standard_normal((40, 12)) * 4
    C, alpha = M.compress_overlap(X, S, 4)
    assert C.shape == (10, 6) and alpha.shape == (10, 8, 6)
    assert np.allclose(alpha.sum(axis=1), 1.0, atol=1e-14)
    assert np.all(alpha[0, 4:] == 0.0) and np.all(alpha[1:] > 0)
    C1, _ = M.compress_overlap(np.full((40, 12), -0.7), S, 4)
    assert np.allclose(C1, -0.7, atol=1e-15)


def test_overlap_without_overlap_logits_is_the_plain_compressor():
    # overlapping-series logits of -inf weight nothing: the primary series alone remains
    rng = np.random.default_rng(21)
    X = rng.standard_normal((32, 10))
    S = rng.standard_normal((32, 10))
    S[:, 5:] = -np.inf
    C, _ = M.compress_overlap(X, S, 4)
    C0, _ = M.compress(X[:, :5], S[:, :5], 4)
    assert np.allclose(C, C0, atol=1e-15)
    # and entry 0 never sees an overlapping token, whatever its logits
    S2 = rng.standard_normal((32, 10))
    Ca, _ = M.compress_overlap(X, S2, 4)
    Cb, _ = M.compress(X[:4, :5], S2[:4, :5], 4)
    assert np.allclose(Ca[0], Cb[0], atol=1e-15)


def test_overlap_ratio_one_closed_form():
    # m = 1: entry i mixes x_A[i] and x_B[i-1] with the weights of a two-way softmax
    rng = np.random.default_rng(22)
    X = rng.standard_normal((9, 4))
    S = rng.standard_normal((9, 4))
    C, _ = M.compress_overlap(X, S, 1)
    assert np.allclose(C[0], X[0, :2])
    for i in range(1, 9):
        sa, sb = S[i, :2], S[i - 1, 2:]
        wa = 1.0 / (1.0 + np.exp(sb - sa))
        assert np.allclose(C[i], wa * X[i, :2] + (1 - wa) * X[i - 1, 2:], atol=1e-14)


def test_overlap_equal_logits_average_the_two_windows():
    rng = np.random.default_rng(23)
    m, d = 4, 3
    X = rng.standard_normal((5 * m, 2 * d))
    S = np.full((5 * m, 2 * d), 0.25)
    C, _ = M.compress_overlap(X, S, m)
    for i in range(1, 5):
        want = np.concatenate([X[m * i: m * i + m, :d], X[m * (i - 1): m * i, d:]]).mean(axis=0)
        assert np.allclose(C[i], want, atol=1e-15)


def test_overlap_boundary_token_feeds_both_neighbouring_entries():
    # a token of block 2 with a dominant primary logit owns entry 2; with a dominant
    # overlapping logit it owns entry 3
    m, d = 4, 2
    X = np.zeros((6 * m, 2 * d))
    X[2 * m + 1] = [1.0, 2.0, 3.0, 4.0]
    S = np.zeros((6 * m, 2 * d))
    S[2 * m + 1, :d] = 80.0
    C, _ = M.compress_overlap(X, S, m)
    assert np.allclose(C[2], [1.0, 2.0], atol=1e-12)
    S = np.zeros((6 * m, 2 * d))
    S[2 * m + 1, d:] = 80.0
    C, _ = M.compress_overlap(X, S, m)
    assert np.allclose(C[3], [3.0, 4.0], atol=1e-12)
    assert np.allclose(C[2], X[2 * m: 3 * m, :d].sum(axis=0) / (2 * m), atol=1e-12)


def test_overlap_positional_encoding_halves():
    # the encoding's first half shifts primary logits, the second half overlapping ones,
    # by the token's place in its block: a per-place constant in the overlapping half moves
    # the overlapping tokens' weights as a logit shift would
    rng = np.random.default_rng(24)
    m, d = 4, 3
    X = rng.standard_normal((6 * m, 2 * d))
    S = rng.standard_normal((6 * m, 2 * d))
    ape = np.zeros((m, 2 * d))
    ape[:, d:] = rng.standard_normal((m, d))
    C1, _ = M.compress_overlap(X, S, m, ape=ape)
    S2 = S.copy()
    S2[:, d:] += np.tile(ape[:, d:], (6, 1))
    C2, _ = M.compress_overlap(X, S2, m)
    assert np.allclose(C1, C2, atol=1e-14)


def test_rms_norm_invariants():
    rng = np.random.default_rng(25)
    x = rng.standard_normal((5, 64)) * 3
    y = M.rms_norm(x, np.ones(64), 0.0)
    assert np.allclose(np.sqrt((y * y).mean(axis=1)), 1.0, atol=1e-14)
    assert np.allclose(M.rms_norm(7.5 * x, np.ones(64), 0.0), y, atol=1e-14)     # scale invariant
    w = rng.standard_normal(64)
    assert np.allclose(M.rms_norm(x, w, 0.0), y * w, atol=1e-14)
    # eps: a zero row stays zero, a tiny row is damped
    assert np.all(M.rms_norm(np.zeros((1, 8)), np.ones(8), 1e-6) == 0.0)


def test_rope_gptj_closed_forms():
    rng = np.random.default_rng(26)
    x = rng.standard_normal((3, 16))
    ones, zeros = np.ones((3, 4)), np.zeros((3, 4))
    assert np.array_equal(M.rope_gptj(x, ones, zeros, 8), x)                 # angle 0
    y = M.rope_gptj(x, zeros, ones, 8)                                         # quarter turn
    assert np.array_equal(y[:, :8], x[:, :8])
    assert np.allclose(y[:, 8::2], -x[:, 9::2]) and np.allclose(y[:, 9::2], x[:, 8::2])
    th1, th2 = rng.uniform(-3, 3, (3, 4)), rng.uniform(-3, 3, (3, 4))
    y1 = M.rope_gptj(M.rope_gptj(x, np.cos(th1), np.sin(th1), 8), np.cos(th2), np.sin(th2), 8)
    y2 = M.rope_gptj(x, np.cos(th1 + th2), np.sin(th1 + th2), 8)
    assert np.allclose(y1, y2, atol=1e-13)                                     # angles add
    yp = y2[:, 8:].reshape(3, 4, 2)
    xp = x[:, 8:].reshape(3, 4, 2)
    assert np.allclose((yp ** 2).sum(-1), (xp ** 2).sum(-1), atol=1e-13)      # pair norms kept


def test_full_compressor_norm_then_rope_at_block_positions():
    # steps 4 and 5 of the pages in that order, RoPE at position m * i of each entry
    rng = np.random.default_rng(27)
    m, d, dr = 4, 16, 8
    X = rng.standard_normal((5 * m, 2 * d))
    S = rng.standard_normal((5 * m, 2 * d))
    w = rng.uniform(0.5, 2.0, d)
    ang = rng.uniform(-3, 3, (64, dr // 2))
    C = M.compress_full(X, S, m, 2, norm_weight=w, eps=1e-6, cos_table=np.cos(ang),
                        sin_table=np.sin(ang), d_rope=dr)
    base, _ = M.compress_overlap(X, S, m)
    normed = M.rms_norm(base, w, 1e-6)
    pos = m * np.arange(5)
    assert np.allclose(C, M.rope_gptj(normed, np.cos(ang[pos]), np.sin(ang[pos]), dr), atol=1e-14)
    # without the epilogue it is the plain entry; coff 1 is compress()
    assert np.allclose(M.compress_full(X, S, m, 2), base)
    assert np.allclose(M.compress_full(X[:, :d], S[:, :d], m, 1), M.compress(X[:, :d], S[:, :d], m)[0])


def _rope_tables(rows: int, d_rope: int, base: float = 10000.0):
    # the standard angle table: pair j of position p turns by p * base^(-2j / d_rope)
    theta = base ** (-2.0 * np.arange(d_rope // 2) / d_rope)
    ang = np.arange(rows)[:, None] * theta[None, :]
    return np.cos(ang), np.sin(ang)


def test_query_and_key_rope_depend_only_on_relative_position():
    # rotating q at p and the KV row at p' leaves their dot product a function of p - p', and
    # rotating both at one position keeps it: the positions index the tables consistently
    rng = np.random.default_rng(28)
    d, dr, H = 32, 16, 3
    cos, sin = _rope_tables(64, dr)
    q = rng.standard_normal((H, d))
    k = rng.standard_normal(d)
    def dots(p, pk):
        return M.qnorm_rope(q, p, cos, sin, dr, 0.0, False) @ M.swa_row(k, pk, cos, sin, dr)
    assert np.allclose(dots(9, 4), dots(30, 25), atol=1e-12)
    assert np.allclose(dots(17, 17), q @ k, atol=1e-12)
    assert not np.allclose(dots(9, 4), dots(9, 5), atol=1e-6)
    # the non-rotated dims are untouched; position 0 is the identity
    assert np.array_equal(M.swa_row(k, 11, cos, sin, dr)[: d - dr], k[: d - dr])
    assert np.allclose(M.swa_row(k, 0, cos, sin, dr), k, atol=0)


def test_query_norm_is_per_head_and_commutes_with_rope():
    rng = np.random.default_rng(29)
    H, d, dr = 4, 32, 8
    cos, sin = _rope_tables(40, dr)
    q = rng.standard_normal((H, d)) * rng.uniform(0.1, 10.0, (H, 1))
    y = M.qnorm_rope(q, 21, cos, sin, dr, 0.0, True)
    assert np.allclose(np.sqrt((y * y).mean(axis=1)), 1.0, atol=1e-14)     # unit RMS per head
    q2 = q.copy()
    q2[1] *= 50.0                                                            # heads independent
    assert np.allclose(M.qnorm_rope(q2, 21, cos, sin, dr, 0.0, True), y, atol=1e-13)
    # the rotation keeps every pair's norm, so norming after it gives the same rows
    r = M.qnorm_rope(q, 21, cos, sin, dr, 0.0, False)
    assert np.allclose(M.rms_norm(r, np.ones(d), 0.0), y, atol=1e-13)
    # no norm and no rotation: the query as given
    assert np.array_equal(M.qnorm_rope(q, 21, None, None, 0, 1e-6, False), q)


def test_indexer_query_and_key_relative_position_and_scales():
    rng = np.random.default_rng(30)
    H, dI, dr, m = 4, 16, 8, 4
    cos, sin = _rope_tables(200, dr)
    q = rng.standard_normal((H, dI))
    kp = rng.standard_normal(dI)
    w = rng.uniform(0, 1, H)
    nw = rng.uniform(0.5, 2.0, dI)
    qr, wr = M.indexer_query(q, 37, cos, sin, dr, w, dI ** -0.5)
    assert np.allclose(wr, w * dI ** -0.5 / 2.0, atol=0)                   # H^-1/2 = 1/2
    # the key is the normed latent, rotated at m * entry: with a query at position p the score
    # depends on p - m * entry only
    def score(p, ent):
        qq, ww = M.indexer_query(q, p, cos, sin, dr, w, 1.0)
        return M.index_scores(qq, ww, M.indexer_key(kp, ent, m, nw, 1e-6, cos, sin, dr)[None])[0]
    assert np.isclose(score(41, 5), score(61, 10), atol=1e-12)              # 41 - 20 = 61 - 40
    assert not np.isclose(score(41, 5), score(41, 6), atol=1e-9)
    k0 = M.indexer_key(kp, 0, m, nw, 1e-6, cos, sin, dr)                   # position 0: no turn
    assert np.allclose(k0, M.rms_norm(kp, nw, 1e-6), atol=0)
    # no rotation on the first dI - dr dims of a key at any entry
    k7 = M.indexer_key(kp, 7, m, nw, 1e-6, cos, sin, dr)
    assert np.array_equal(k7[: dI - dr], k0[: dI - dr])


def test_candidate_blocks_reduce_to_topk_and_block_max():
    rng = np.random.default_rng(40)
    sc = rng.standard_normal(103)
    # blocks of one entry: the candidate blocks are the plain top-k
    assert np.array_equal(M.candidate_blocks(sc, 1, 17), M.topk(sc, 17))
    # brute force over blocks of 8 (the last one ragged): sort by (-max, id)
    bm = [(-sc[b * 8:(b + 1) * 8].max(), b) for b in range(13)]
    want = [b for _, b in sorted(bm)][:5]
    assert list(M.candidate_blocks(sc, 8, 5)) == want
    # fewer blocks than asked: all of them, -1 padded
    got = M.candidate_blocks(sc, 64, 4)
    assert sorted(got[:2].tolist()) == [0, 1] and list(got[2:]) == [-1, -1]
    # equal block maxima: the smaller block id first
    eq = np.zeros(32)
    assert list(M.candidate_blocks(eq, 8, 2)) == [0, 1]


def test_topk_in_blocks_restricts_the_selection():
    rng = np.random.default_rng(41)
    sc = rng.standard_normal(300)
    # every block listed: the plain top-k
    assert np.array_equal(M.topk_in_blocks(sc, list(range(10)), 32, 40), M.topk(sc, 40))
    blocks = [7, 2, -1, 9]
    got = M.topk_in_blocks(sc, blocks, 32, 20)
    inside = np.array([e for b in (2, 7, 9) for e in range(32 * b, min(300, 32 * b + 32))])
    assert set(got.tolist()) <= set(inside.tolist())
    assert sc[inside].max() == sc[got].max()
    assert np.all(sc[np.setdiff1d(inside, got)] <= sc[got].min())
    # fewer entries than k (block 9 holds 12 visible entries): all selected, -1 padded
    got = M.topk_in_blocks(sc, [9], 32, 20)
    assert sorted(got[:12].tolist()) == list(range(288, 300)) and np.all(got[12:] == -1)
    # the two levels together with blocks of one entry: the consumer's top-k is the source's
    src = M.candidate_blocks(sc, 1, 40)
    assert set(M.topk_in_blocks(sc, src, 1, 40).tolist()) == set(M.topk(sc, 40).tolist())


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
