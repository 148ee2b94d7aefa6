"""hcs_sparse_mla_decode_noalloc (the decode attention with the library's static scratch, for
callers that cannot allocate) against hcs_sparse_mla_decode with a workspace, through the C ABI
(MI355X only): the same plan and kernels, so the same bits, on two calls in a row, the second
with a smaller input; and parity with the oracle on a few queries."""
import numpy as np
import pytest
import torch

import hybrid_compressed_sparse_amd as hcs
from hybrid_compressed_sparse_amd.step import PathStep
from oracle import pipeline as OP
from synth import configs as C
from synth import gen as G

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests import gpu_util as U


def _dev():
    return torch.device("cuda:0")


def _selection(sc):
    """The indexer's top-k (CSA) or None (HCA), after the step's compressor ran."""
    step, _ = U.run_step(sc)
    return step.idx if sc.wl.indexer else None


def _both(sc, idx):
    wl = sc.wl
    outs = []
    for noalloc in (False, True):
        out = torch.full((sc.N, wl.H, wl.d), float("nan"), dtype=torch.bfloat16, device=_dev())
        lse = torch.full((sc.N, wl.H), float("nan"), dtype=torch.float32, device=_dev())
        args = (sc.q, sc.swa, sc.comp, idx, sc.q_seq, sc.q_pos, wl.window, wl.m, sc.max_pos(), wl.d ** -0.5, out, lse)
        if noalloc:
            hcs.sparse_mla_decode_noalloc(*args)
        else:
            hcs.sparse_mla_decode(*args)
        torch.cuda.synchronize()
        outs.append((out, lse))
    return outs


@pytest.mark.parametrize("case", ["csa", "hca", "fp8"])
def test_noalloc_matches_workspace_entry_point(case):
    if case == "csa":
        big = G.build(C.CSA_DECODE, seed=41, device=_dev())
        small = G.build(C.CSA_DECODE.with_(B=5, topk=300), seed=42, device=_dev(),
                        ctx_per_seq=[8192, 5000, 2047, 640, 77])
    elif case == "hca":
        big = G.build(C.HCA_DECODE, seed=43, device=_dev())
        small = G.build(C.HCA_DECODE.with_(B=3), seed=44, device=_dev(), ctx_per_seq=[131072, 70000, 300])
    else:
        big = G.build(C.CSA_DECODE_1M_FP8.with_(B=4), seed=45, device=_dev(), ctx_per_seq=[1 << 20] * 4)
        small = G.build(C.CSA_DECODE_1M_FP8.with_(B=2, topk=256), seed=46, device=_dev(),
                        ctx_per_seq=[65536, 9000])
    for sc in (big, small):                            # two calls in a row, the second smaller
        U.say(f"[case] noalloc {case} {sc.wl.name} N={sc.N} seed={sc.seed}")
        idx = _selection(sc)
        (o1, l1), (o2, l2) = _both(sc, idx)
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
        assert torch.equal(l1, l2)
        qs = [0, sc.N - 1]
        sel = None
        if sc.wl.indexer:
            sel = {t: idx[t].cpu().numpy() for t in qs}
        ref = OP.step(sc, queries=qs, selected_override=sel)
        for t in qs:
            U.check_attention(o2[t].float().cpu().numpy().astype(np.float64), ref["o"][t], sc.wl.kv_fmt,
                              l2[t].double().cpu().numpy(), ref["lse"][t])
