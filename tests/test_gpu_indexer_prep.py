"""Parity of the indexer query and key production (hcs_indexer_q_prep, hcs_indexer_k_store) with
the oracle's indexer_query / indexer_key and its MXFP4 / FP8 encoders, and of the FP8 (132-byte)
key scoring with the oracle's scores over the stored codes."""
import numpy as np
import pytest
import torch

import hybrid_compressed_sparse_amd as hcs
from oracle import formats as OF
from oracle import method as OM
from oracle import pipeline as OP
from synth import layout as L

import gpu_util as U

pytestmark = pytest.mark.gpu

DI, DR = 128, 64


def _dev():
    return torch.device("cuda:0")


def _tables(rows):
    theta = 10000.0 ** (-2.0 * torch.arange(DR // 2, dtype=torch.float64) / DR)
    ang = torch.arange(rows, dtype=torch.float64)[:, None] * theta[None, :]
    return torch.cos(ang).float(), torch.sin(ang).float()


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _nibbles(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def _e2m1_step(ref, e):
    # spacing of e2m1 around |ref| / 2^e (0.5 below 2, 1 up to 4, 2 above), in value units
    y = np.abs(ref) / np.ldexp(1.0, e)
    return np.where(y < 2.0, 0.5, np.where(y < 4.0, 1.0, 2.0)) * np.ldexp(1.0, e)


def _check_quantized(fmt, ref, got_codes, got_scale):
    """ref float64 [R, 128]; the GPU's codes / scales against the oracle's encoding of ref in
    float32 (the precision both sides decide the codes in, up to rounding order)."""
    if fmt == "mxfp4":
        packed, sc = OF.quantize_mxfp4(ref.astype(np.float32))
        same = (_nibbles(got_codes) == _nibbles(packed)).mean()
        assert same >= 0.999, same
        assert (got_scale == sc).mean() >= 0.999
        dec = OF.decode_mxfp4(got_codes, got_scale)
        e = np.repeat(sc.astype(np.int64) - 127, 32, axis=-1)
        assert np.all(np.abs(dec - ref) <= _e2m1_step(ref, e))
    else:
        codes, sc = OF.quantize_fp8ix(ref.astype(np.float32))
        assert (got_codes == codes).mean() >= 0.999
        assert (got_scale == sc).mean() >= 0.999
        dec = OF.decode_fp8ix(got_codes, got_scale)
        lim = np.abs(ref) * 2.0 ** -3 + 2.0 ** -9 * sc[:, None].astype(np.float64)
        assert np.all(np.abs(dec - ref) <= lim)


def _q_inputs(seed, N, H):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(N, H, DI, generator=g).to(torch.bfloat16)
    w = torch.rand(N, H, generator=g)
    pos = torch.randint(0, 3000, (N,), generator=g, dtype=torch.int32)
    return q, w, pos


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "fp8ix"])
@pytest.mark.parametrize("H", [64, 20])
def test_indexer_query_matches_oracle(fmt, H):
    N = 37
    q, w, pos = _q_inputs(21 + H, N, H)
    pos[4] = -1                                             # skipped token
    cos, sin = _tables(3000)
    dev = _dev()
    w_scale = DI ** -0.5 * H ** -0.5
    if fmt == "bf16":
        q_out = torch.full((N, H, DI), 7.0, dtype=torch.bfloat16, device=dev)
        q_sc = None
    elif fmt == "mxfp4":
        q_out = torch.full((N, H, DI // 2), 0xAB, dtype=torch.uint8, device=dev)
        q_sc = torch.full((N, H, 4), 0xCD, dtype=torch.uint8, device=dev)
    else:
        q_out = torch.full((N, H, DI), 0xAB, dtype=torch.uint8, device=dev)
        q_sc = torch.full((N, H), -1.0, dtype=torch.float32, device=dev)
    w_out = torch.full((N, H), -1.0, dtype=torch.float32, device=dev)
    hcs.indexer_q_prep(q.to(dev), w.to(dev), pos.to(dev), fmt, q_out, w_out, q_sc, w_scale=w_scale,
                       rope_cos=cos.to(dev), rope_sin=sin.to(dev))
    torch.cuda.synchronize()
    q64 = OP.decode_input(q)
    c64, s64 = cos.double().numpy(), sin.double().numpy()
    wo = w_out.cpu().numpy()
    qo = q_out.cpu()
    so = None if q_sc is None else q_sc.cpu().numpy()
    for t in range(N):
        if pos[t] < 0:
            assert np.all(wo[t] == -1.0)
            if fmt == "bf16":
                assert torch.all(qo[t].float() == 7.0)
            else:
                assert torch.all(qo[t] == 0xAB)
            continue
        ref, wr = OM.indexer_query(q64[t], int(pos[t]), c64, s64, DR, w[t].double().numpy(), DI ** -0.5)
        assert np.allclose(wo[t], wr, rtol=2e-7, atol=0)
        if fmt == "bf16":
            got = OF.decode_bf16(_bits(qo[t]))
            _, e = np.frexp(np.abs(ref))
            assert np.all(np.abs(got - ref) <= np.ldexp(1.0, e - 8) + 1e-6)
        else:
            _check_quantized(fmt, ref, qo[t].numpy(), so[t])


def _key_cache(seed, n_seq, n_ent, fmt):
    n_pg = (n_ent + 63) // 64
    g = torch.Generator().manual_seed(seed)
    pt = torch.randperm(n_seq * n_pg, generator=g).to(torch.int32).view(n_seq, n_pg).clone()
    pool = L.new_pool(n_seq * n_pg, fmt, DI, "cpu")
    pool.copy_(torch.randint(0, 256, pool.shape, generator=g, dtype=torch.uint8))
    return pool.to(_dev()), pt.to(_dev())


def _store_all_keys(seed, n_seq, n_ent, m, fmt, drop=None):
    """Keys of entries 0..n_ent-1 of every sequence, written by hcs_indexer_k_store in a shuffled
    row order. Returns (pool, page table, k_pre, norm weight, tables, entry seq / idx)."""
    g = torch.Generator().manual_seed(seed)
    k_pre = (torch.randn(n_seq * n_ent, DI + 32, generator=g) * 2).to(torch.bfloat16)
    nw = torch.rand(DI, generator=g) + 0.5
    perm = torch.randperm(n_seq * n_ent, generator=g)
    ent_seq = (perm // n_ent).to(torch.int32)
    ent_idx = (perm % n_ent).to(torch.int32)
    if drop is not None:
        ent_idx[drop] = -1
    cos, sin = _tables(m * n_ent + 1)
    pool, pt = _key_cache(seed, n_seq, n_ent, fmt)
    dev = _dev()
    kd = k_pre.to(dev)
    hcs.indexer_k_store(kd[:, :DI], ent_seq.to(dev), ent_idx.to(dev), m, hcs.paged(pool, pt, fmt, DI),
                        nw.to(dev), eps=1e-6, rope_cos=cos.to(dev), rope_sin=sin.to(dev))
    torch.cuda.synchronize()
    return pool, pt, k_pre, nw, cos, sin, ent_seq, ent_idx


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "fp8ix"])
def test_indexer_keys_match_oracle(fmt):
    n_seq, n_ent, m = 3, 150, 4
    pool, pt, k_pre, nw, cos, sin, ent_seq, ent_idx = _store_all_keys(31, n_seq, n_ent, m, fmt, drop=[7, 8])
    k64 = OP.decode_input(k_pre[:, :DI])
    c64, s64 = cos.double().numpy(), sin.double().numpy()
    pool_before, _ = _key_cache(31, n_seq, n_ent, fmt)      # the same pre-fill
    for r in range(k_pre.shape[0]):
        b, i = int(ent_seq[r]), int(ent_idx[r])
        if i < 0:
            continue
        ref = OM.indexer_key(k64[r], i, m, nw.double().numpy(), 1e-6, c64, s64, DR)
        row = L.gather_rows(pool, fmt, DI, pt[b], torch.tensor([i]))
        if fmt == "bf16":
            got = OF.decode_bf16(_bits(row))[0]
            _, e = np.frexp(np.abs(ref))
            assert np.all(np.abs(got - ref) <= np.ldexp(1.0, e - 8) + 1e-6), r
        elif fmt == "mxfp4":
            _check_quantized(fmt, ref[None], row.codes.cpu().numpy(), row.scales.cpu().numpy())
        else:
            _check_quantized(fmt, ref[None], row.codes.cpu().numpy(), row.scale.cpu().numpy())
    # every row nobody wrote (including the entries of the rows with index -1) keeps its bytes
    written = torch.zeros(n_seq, ((n_ent + 63) // 64) * 64, dtype=torch.bool)
    for r in range(k_pre.shape[0]):
        if int(ent_idx[r]) >= 0:
            written[int(ent_seq[r]), int(ent_idx[r])] = True
    for b in range(n_seq):
        ids = torch.nonzero(~written[b]).flatten()
        old = L.gather_rows(pool_before, fmt, DI, pt[b], ids)
        new = L.gather_rows(pool, fmt, DI, pt[b], ids)
        if fmt == "bf16":
            assert torch.equal(old.view(torch.int16), new.view(torch.int16))
        elif fmt == "mxfp4":
            assert torch.equal(old.codes, new.codes) and torch.equal(old.scales, new.scales)
        else:
            assert torch.equal(old.codes, new.codes)
            assert torch.equal(old.scale.view(torch.int32), new.scale.view(torch.int32))


@pytest.mark.parametrize("n_ent,topk", [(700, 128), (90, 128)], ids=["select", "short_context"])
def test_fp8_key_scores_and_topk(n_ent, topk):
    """Queries and keys made by the two calls above, scored from the 132-byte FP8 rows; the
    oracle scores the stored codes (decoded) with the returned weights."""
    n_seq, m, H, N = 2, 4, 64, 12
    pool, pt, *_ = _store_all_keys(41, n_seq, n_ent, m, "fp8ix")
    g = torch.Generator().manual_seed(42)
    q = torch.randn(N, H, DI, generator=g).to(torch.bfloat16)
    w = torch.rand(N, H, generator=g)
    q_seq = torch.randint(0, n_seq, (N,), generator=g, dtype=torch.int32)
    q_pos = torch.randint(0, m * n_ent, (N,), generator=g, dtype=torch.int32)
    q_pos[0] = m * n_ent - 1
    cos, sin = _tables(m * n_ent + 1)
    dev = _dev()
    q_codes = torch.empty((N, H, DI), dtype=torch.uint8, device=dev)
    q_sc = torch.empty((N, H), dtype=torch.float32, device=dev)
    w_out = torch.empty((N, H), dtype=torch.float32, device=dev)
    hcs.indexer_q_prep(q.to(dev), w.to(dev), q_pos.to(dev), "fp8ix", q_codes, w_out, q_sc,
                       w_scale=DI ** -0.5 * H ** -0.5, rope_cos=cos.to(dev), rope_sin=sin.to(dev))
    out_idx = torch.empty((N, topk), dtype=torch.int32, device=dev)
    out_score = torch.empty((N, topk), dtype=torch.float32, device=dev)
    max_pos = m * n_ent - 1
    hcs.index_topk(q_codes, q_sc, w_out, hcs.paged(pool, pt, "fp8ix", DI), q_seq.to(dev), q_pos.to(dev), m,
                   topk, max_pos, out_idx, out_score)
    torch.cuda.synchronize()
    qd = OF.decode_fp8ix(q_codes.cpu().numpy(), q_sc.cpu().numpy())
    wd = w_out.cpu().numpy().astype(np.float64)
    for t in range(N):
        b, p = int(q_seq[t]), int(q_pos[t])
        nv = OM.n_visible(p, m)
        rows = L.gather_rows(pool, "fp8ix", DI, pt[b], torch.arange(nv))
        K = OF.decode_fp8ix(rows.codes.cpu().numpy(), rows.scale.cpu().numpy())
        sc = OM.index_scores(qd[t], wd[t], K)
        ref = OM.topk(sc, topk)
        U.check_topk(out_idx[t].cpu().numpy(), out_score[t].cpu().numpy(), ref, sc, topk)
