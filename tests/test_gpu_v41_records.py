"""The V4.1 cache records on the GPU: MXFP8 window and compressed rows (528 bytes) and NVFP4
compressed rows (288 bytes), written by the compressor and the window insert and read by the
decode attention, against the oracle (MI355X only)."""
import numpy as np
import pytest
import torch

import hybrid_compressed_sparse_amd as hcs
from oracle import formats as OF
from oracle import method as OM
from oracle import pipeline as OP
from synth import configs as C
from synth import gen as G
from synth import layout as L

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as U
    from tests.test_gpu_parity import _check_step
    from tests import test_gpu_compressor_full as CF


def _dev():
    return torch.device("cuda:0")


@pytest.mark.parametrize("comp_fmt", ["mxfp8", "nvfp4"])
def test_v41_decode_step_small(comp_fmt):
    """The whole CSA decode step (compressor store, MXFP4 indexer, attention) with MXFP8 window
    rows and MXFP8 or NVFP4 compressed rows; ragged contexts, some not ending a block."""
    wl = C.CSA_DECODE_1M_FP8.with_(B=3, topk=256, kv_fmt="mxfp8", comp_fmt=comp_fmt)
    sc = G.build(wl, seed=61, device=_dev(), ctx_per_seq=[65536, 20001, 902])
    _check_step(sc)


def test_v41_hca_decode_nvfp4_all_entries():
    """HCA over every visible NVFP4 entry (no indexer), MXFP8 window rows."""
    wl = C.HCA_DECODE.with_(B=4, kv_fmt="mxfp8", comp_fmt="nvfp4")
    sc = G.build(wl, seed=62, device=_dev(), ctx_per_seq=[131072, 50000, 129, 4096])
    _check_step(sc)


@pytest.mark.parametrize("fmt", ["mxfp8", "nvfp4"])
def test_v41_full_compressor_store(fmt):
    """The full compressor (overlap, RMSNorm, RoPE) storing MXFP8 / NVFP4 entries."""
    lens, d, m, coff, dr = [2049, 777, 1], 512, 4, 2, 64
    X, S, ape, w, cos, sin = CF._inputs(63, lens, d, m, coff, False, True, dr)
    pool, pt, state, dbg, starts = CF._run(X, S, ape, w, cos, sin, lens, d, m, coff, fmt, [], 63)
    ref = CF._oracle(X, S, ape, w, cos, sin, m, coff, dr)
    for b, Cb in enumerate(ref):
        n = Cb.shape[0]
        if n == 0:
            continue
        rows = L.gather_rows(pool, fmt, d, pt[b], torch.arange(n, device=pool.device))
        U.check_v41_rows(fmt, rows, Cb)


def test_v41_window_insert_mxfp8():
    """hcs_qnorm_rope_kv_insert into an MXFP8 window cache: codes and scales of the blocks the
    rotation does not touch are exact (the float32 values are the bf16 inputs); the rotated
    blocks agree with the oracle to the rounding bar."""
    d, B, max_pos = 512, 2, 300
    g = torch.Generator().manual_seed(64)
    seq = torch.arange(B, dtype=torch.int32).repeat_interleave(50)
    pos = torch.cat([torch.randperm(max_pos, generator=g)[:50] for _ in range(B)]).to(torch.int32)
    kv = (torch.randn(seq.shape[0], d, generator=g) * 0.3).to(torch.bfloat16)
    theta = 10000.0 ** (-2.0 * torch.arange(32, dtype=torch.float64) / 64)
    ang = torch.arange(max_pos, dtype=torch.float64)[:, None] * theta[None, :]
    cos, sin = torch.cos(ang).float(), torch.sin(ang).float()
    n_pg = (max_pos + 63) // 64
    pt = torch.randperm(B * n_pg, generator=g).to(torch.int32).view(B, n_pg)
    dev = _dev()
    pool = L.new_pool(B * n_pg, "mxfp8", d, dev)
    ptd = pt.to(dev)                 # held: the paged descriptor keeps only its address
    hcs.qnorm_rope_kv_insert(None, kv.to(dev), seq.to(dev), pos.to(dev), hcs.paged(pool, ptd, "mxfp8", d),
                             rope_cos=cos.to(dev), rope_sin=sin.to(dev), d=d)
    torch.cuda.synchronize()
    kv64 = OP.decode_input(kv)
    ref = np.stack([OM.swa_row(kv64[t], int(pos[t]), cos.double().numpy(), sin.double().numpy(), 64)
                    for t in range(seq.shape[0])])
    got = [L.gather_rows(pool, "mxfp8", d, ptd[b], pos[seq == b].long()) for b in range(B)]
    rc, rs = OF.quantize_mxfp8(ref.astype(np.float32))
    codes = np.concatenate([r.codes.cpu().numpy() for r in got])
    scales = np.concatenate([r.scales.cpu().numpy() for r in got])
    order = np.concatenate([np.nonzero(seq.numpy() == b)[0] for b in range(B)])
    rc, rs = rc[order], rs[order]
    assert np.array_equal(codes[:, :448], rc[:, :448]) and np.array_equal(scales[:, :14], rs[:, :14])
    assert (codes[:, 448:] == rc[:, 448:]).mean() >= 0.999
    U.check_v41_rows("mxfp8", L.Mxfp4Rows(torch.from_numpy(codes), torch.from_numpy(scales)), ref[order])
