"""Parity of the query preparation and sliding-window insert (hcs_qnorm_rope_kv_insert) with the
oracle's qnorm_rope and swa_row, on seeded synthetic tokens: several sequences, positions that
cross page boundaries, non-resident pages and skipped tokens; then a decode attention over the
inserted rows."""
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


def _tokens(seed, B, per_seq, d, H, max_pos, d_rope):
    """Tokens of B sequences (per_seq each, distinct positions in [0, max_pos)), their q heads,
    KV rows and the RoPE tables (the standard angle table of base 10000)."""
    g = torch.Generator().manual_seed(seed)
    seq, pos = [], []
    for b in range(B):
        p = torch.randperm(max_pos, generator=g)[:per_seq].sort().values
        seq += [b] * per_seq
        pos += p.tolist()
    N = len(pos)
    q = (torch.randn(N, H, d, generator=g) * torch.rand(N, H, 1, generator=g) * 4).to(torch.bfloat16)
    kv = (torch.randn(N, d, generator=g) * 0.3).to(torch.bfloat16)
    theta = 10000.0 ** (-2.0 * torch.arange(d_rope // 2, dtype=torch.float64) / d_rope)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * theta[None, :]
    return (torch.tensor(seq, dtype=torch.int32), torch.tensor(pos, dtype=torch.int32), q, kv,
            torch.cos(ang).float(), torch.sin(ang).float())


def _swa(seed, B, max_pos, d, fmt, drop_page=None):
    """A sliding-window cache covering positions [0, max_pos) of every sequence in shuffled pages,
    pre-filled with a byte pattern; drop_page = (b, j) makes page j of sequence b non-resident."""
    n_pg = (max_pos + 63) // 64
    g = torch.Generator().manual_seed(seed + 7)
    perm = torch.randperm(B * n_pg, generator=g).to(torch.int32)
    pt = perm.view(B, n_pg).clone()
    if drop_page is not None:
        pt[drop_page] = -1
    pool = L.new_pool(B * n_pg, fmt, d, "cpu")
    pool.copy_(torch.randint(0, 256, pool.shape, generator=g, dtype=torch.uint8))
    if fmt == "fp8ds":   # keep the pre-fill decodable: scale bytes near 127
        v = L._region_views(pool, fmt, d)[2]
        v.copy_(torch.randint(120, 130, v.shape, generator=g, dtype=torch.uint8))
    return pool.to(_dev()), pt.to(_dev())


def _bf16_close(got, ref):
    # within one bf16 step of the reference, plus a float32-sized allowance on the row's scale
    _, e = np.frexp(np.abs(ref))
    lim = np.ldexp(1.0, e - 8) + 1e-5 * np.abs(ref).max(axis=-1, keepdims=True)
    return np.abs(got - ref) <= lim


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("d,H,q_norm", [(512, 64, False), (512, 6, True), (128, 8, True), (128, 13, False)],
                         ids=["d512_h64", "d512_h6_norm", "d128_h8_norm", "d128_h13"])
def test_query_preparation_matches_oracle(d, H, q_norm):
    seq, pos, q, kv, cos, sin = _tokens(11, 3, 37, d, H, 300, 64)
    dev = _dev()
    qd = q.to(dev)
    hcs.qnorm_rope_kv_insert(qd, None, None, pos.to(dev), rope_cos=cos.to(dev), rope_sin=sin.to(dev),
                             q_norm=q_norm, eps=1e-6)
    torch.cuda.synchronize()
    got = OF.decode_bf16(_bits(qd.cpu()))
    q64 = OP.decode_input(q)
    for t in range(pos.shape[0]):
        ref = OM.qnorm_rope(q64[t], int(pos[t]), cos.double().numpy(), sin.double().numpy(), 64, 1e-6, q_norm)
        ok = _bf16_close(got[t], ref)
        assert ok.all(), (t, int(pos[t]), np.abs(got[t] - ref).max())


@pytest.mark.parametrize("fmt", ["bf16", "fp8ds"])
def test_swa_insert_matches_oracle(fmt):
    d, H, B, max_pos = 512, 4, 3, 200
    seq, pos, q, kv, cos, sin = _tokens(12, B, 45, d, H, max_pos, 64)
    pos[5] = -1                                              # a skipped token
    dev = _dev()
    pool, pt = _swa(12, B, max_pos, d, fmt, drop_page=(1, 2))   # positions 128..191 of seq 1
    before = pool.clone()
    # kv rows with a wider stride (the first d columns are the row)
    kv_wide = torch.zeros(kv.shape[0], d + 64, dtype=torch.bfloat16)
    kv_wide[:, :d] = kv
    kvd = kv_wide.to(dev)
    qd = q.to(dev)
    hcs.qnorm_rope_kv_insert(qd, kvd[:, :d], seq.to(dev), pos.to(dev), hcs.paged(pool, pt, fmt, d),
                             rope_cos=cos.to(dev), rope_sin=sin.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(kvd.cpu(), kv_wide)                   # the KV input is not modified
    assert torch.equal(qd[5].cpu().view(torch.int16), q[5].view(torch.int16))   # skipped token
    kv64 = OP.decode_input(kv)
    written = torch.zeros(B, max_pos, dtype=torch.bool)
    for t in range(pos.shape[0]):
        b, p = int(seq[t]), int(pos[t])
        if p < 0 or (b == 1 and 128 <= p < 192):
            continue
        written[b, p] = True
        ref = OM.swa_row(kv64[t], p, cos.double().numpy(), sin.double().numpy(), 64)
        row = L.gather_rows(pool, fmt, d, pt[b], torch.tensor([p]))
        if fmt == "bf16":
            got = OF.decode_bf16(_bits(row))[0]
            assert _bf16_close(got, ref).all(), (t, p)
        else:
            codes, rope_bits, scales = OF.quantize_fp8ds(ref[None].astype(np.float32))
            # the latent dims are not rotated: the float32 values are the bf16 inputs, so the
            # scale and every code are exact
            assert np.array_equal(row.codes.cpu().numpy(), codes), (t, p)
            assert np.array_equal(row.scales.cpu().numpy(), scales), (t, p)
            gr = OF.decode_bf16(_bits(row.rope))[0]
            assert _bf16_close(gr, ref[448:]).all(), (t, p)
    # nothing else changed: rows not written keep their bytes (pad bytes of written rows are 0)
    for b in range(B):
        ids = torch.nonzero(~written[b]).flatten()
        ids = ids[(pt[b].cpu()[ids // 64] >= 0)]
        old = L.gather_rows(before, fmt, d, pt[b], ids)
        new = L.gather_rows(pool, fmt, d, pt[b], ids)
        if fmt == "bf16":
            assert torch.equal(old.view(torch.int16), new.view(torch.int16))
        else:
            assert torch.equal(old.codes, new.codes) and torch.equal(old.scales, new.scales)
            assert torch.equal(old.rope.view(torch.int16), new.rope.view(torch.int16))
    if fmt == "fp8ds":
        pad = L._region_views(pool, fmt, d)[2][..., 7].cpu()
        for b in range(B):
            for p in torch.nonzero(written[b]).flatten().tolist():
                assert int(pad[pt[b, p // 64].item(), p % 64]) == 0


def test_insert_then_window_attention():
    # rows inserted by the call are the rows the decode attention reads at their positions
    d, H, B, max_pos, window = 512, 16, 2, 256, 128
    g = torch.Generator().manual_seed(13)
    dev = _dev()
    pool, pt = _swa(13, B, max_pos, d, "bf16")
    # every position of both sequences gets a row through the insert
    seq = torch.arange(B, dtype=torch.int32).repeat_interleave(max_pos)
    pos = torch.arange(max_pos, dtype=torch.int32).repeat(B)
    kv = (torch.randn(B * max_pos, d, generator=g) * 0.3).to(torch.bfloat16)
    q = torch.randn(B * max_pos, H, d, generator=g).to(torch.bfloat16)
    theta = 10000.0 ** (-2.0 * torch.arange(32, dtype=torch.float64) / 64)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * theta[None, :]
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    qd = q.to(dev)
    swa = hcs.paged(pool, pt, "bf16", d)
    hcs.qnorm_rope_kv_insert(qd, kv.to(dev), seq.to(dev), pos.to(dev), swa, rope_cos=cos.to(dev),
                             rope_sin=sin.to(dev), q_norm=True, eps=1e-6)
    # decode queries: the last token of each sequence and one in the middle; m larger than any
    # position, so no compressed entry is visible and only the window is attended
    pick = [max_pos - 1, 70, max_pos + max_pos - 1, max_pos + 130]
    qs = qd[pick].contiguous()
    q_seq = seq[pick].to(dev)
    q_pos = pos[pick].to(dev)
    comp_pool = L.new_pool(1, "bf16", d, dev)
    comp_pt = torch.zeros((B, 1), dtype=torch.int32, device=dev)
    comp = hcs.paged(comp_pool, comp_pt, "bf16", d)
    out = torch.empty_like(qs)
    m = 1024
    hcs.sparse_mla_decode(qs, swa, comp, None, q_seq, q_pos, window=window, m=m, max_pos=max_pos - 1,
                          scale=1.0 / math.sqrt(d), out=out)
    torch.cuda.synchronize()
    kv64 = OP.decode_input(kv)
    q64 = OP.decode_input(q)
    c64, s64 = cos.double().numpy(), sin.double().numpy()
    got = OF.decode_bf16(_bits(out.cpu()))
    for i, t in enumerate(pick):
        b, p = int(seq[t]), int(pos[t])
        lo = max(0, p - window + 1)
        rows = np.stack([OM.swa_row(kv64[b * max_pos + r], r, c64, s64, 64) for r in range(lo, p + 1)])
        rows = OF.decode_bf16(OF.round_bf16(rows))          # the cache holds bf16 rows
        qr = OF.decode_bf16(OF.round_bf16(OM.qnorm_rope(q64[t], p, c64, s64, 64, 1e-6, True)))
        ref, _ = OM.attention(qr, rows, 1.0 / math.sqrt(d))
        assert np.abs(got[i] - ref).max() <= 2e-2, (i, np.abs(got[i] - ref).max())
