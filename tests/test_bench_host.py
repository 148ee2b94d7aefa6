"""Host-side parts of bench.py (no GPU): the algorithmic bytes of each decode workload agree with
the per-step figures derived from the configurations' shapes, and the percentile helper."""
import pytest

import bench
from synth import configs as C


@pytest.mark.parametrize("wl, mb", [(C.CSA_DECODE, 43.10), (C.HCA_DECODE, 84.87), (C.CSA_DECODE_1M_FP8, 154.24)])
def test_algorithmic_bytes_per_step(wl, mb):
    # the figures count q, the window and selected rows, ids, out, the indexer keys scanned, the
    # compressor's state and one token; page-table accounting differs by well under 1%
    got = bench.algo_bytes(wl, wl.ctx // wl.m)["step"] / 1e6
    assert abs(got - mb) <= 0.01 * mb, got


def test_attention_bytes_csa_decode():
    # per query: q 64 KiB, 128 window rows + 512 selected rows of 1 KiB, ids, out 64 KiB, lse
    b = bench.algo_bytes(C.CSA_DECODE, 2048)["attention"] / C.CSA_DECODE.B
    assert 65536 + 640 * 1024 + 512 * 4 + 65536 + 256 <= b <= 65536 + 640 * 1024 + 512 * 4 + 65536 + 256 + 400


def test_percentiles_nearest_rank():
    st = bench.pct_stats([float(x) for x in range(100, 0, -1)])
    assert (st["p10_ms"], st["p50_ms"], st["p90_ms"], st["samples"]) == (10.0, 50.0, 90.0, 100)
    assert bench.pct_stats([3.0])["p90_ms"] == 3.0
