"""The five workload shapes of the hot path.

Each workload is one step of the path: the KV compressor on the step's new
tokens, the Lightning-Indexer top-k (CSA layers only) and single-KV-head sparse
MLA attention over the sliding window plus the compressed entries.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "decode" (one query per sequence), "tiny" or "prefill"
    B: int               # sequences
    ctx: int             # decode: tokens in each sequence after this step (query at ctx-1)
    H: int               # query heads sharing the one KV head
    d: int               # head dim (last d_rope dims rotary)
    d_rope: int
    m: int               # compression ratio
    window: int          # sliding-window rows, the query's own token included
    indexer: bool        # CSA (top-k over compressed entries) vs HCA (all of them)
    H_I: int = 0         # indexer heads
    d_I: int = 0         # indexer dim
    topk: int = 0
    kv_fmt: str = "bf16"     # window rows (and compressed rows unless comp_fmt is set): "bf16",
                             # "fp8ds" (584 B per row) or "mxfp8" (528 B per row)
    comp_fmt: str = ""       # compressed rows when they differ: "nvfp4" (288 B per row)
    ix_fmt: str = "bf16"     # "bf16" or "mxfp4" (e2m1 + UE8M0 per 32)
    in_dtype: str = "f32"    # compressor input dtype ("bf16" or "f32")
    P0: int = 0              # prefill: absolute position of the first new token
    Q: int = 0               # prefill: new tokens (= queries) in the chunk
    n_query: int = 0         # tiny: decode queries at the end of the one sequence
    q_std: float = 0.0       # std of q (and indexer q); 0 -> 1/sqrt(dim)

    @property
    def cfmt(self) -> str:
        return self.comp_fmt or self.kv_fmt

    @property
    def n_queries(self) -> int:
        if self.kind == "decode":
            return self.B
        if self.kind == "prefill":
            return self.Q
        return self.n_query

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# One sequence of 1024 tokens, 4 decode queries at its end; checkable on the CPU.
TINY_CSA = Workload(
    name="tiny_csa", kind="tiny", B=1, ctx=1024, H=8, d=128, d_rope=32, m=4, window=16,
    indexer=True, H_I=4, d_I=32, topk=32, in_dtype="bf16", n_query=4, q_std=1.0)

# CSA decode: 32 sequences at 8192 tokens, k=512 of 2048 compressed entries.
CSA_DECODE = Workload(
    name="csa_decode_bf16", kind="decode", B=32, ctx=8192, H=64, d=512, d_rope=64, m=4,
    window=128, indexer=True, H_I=64, d_I=128, topk=512)

# HCA decode: 64 sequences at 131072 tokens, all 1024 compressed entries attended.
HCA_DECODE = Workload(
    name="hca_decode_bf16", kind="decode", B=64, ctx=131072, H=64, d=512, d_rope=64, m=128,
    window=128, indexer=False)

# CSA prefill chunk: 4096 new tokens after a 65536-token prefix, k=2048 per query.
CSA_PREFILL = Workload(
    name="csa_prefill_bf16", kind="prefill", B=1, ctx=65536 + 4096, H=64, d=512, d_rope=64,
    m=4, window=128, indexer=True, H_I=64, d_I=128, topk=2048, P0=65536, Q=4096)

# CSA decode at 1M context: fp8_ds KV (e4m3 + UE8M0 per 64 on 448 latent dims, bf16 rope)
# and MXFP4 indexer keys/queries, k=2048 of 262144 compressed entries.
CSA_DECODE_1M_FP8 = Workload(
    name="csa_decode_1m_fp8", kind="decode", B=8, ctx=1048576, H=64, d=512, d_rope=64, m=4,
    window=128, indexer=True, H_I=64, d_I=128, topk=2048, kv_fmt="fp8ds", ix_fmt="mxfp4")

# The same with the V4.1 records: MXFP8 window rows (528 B), NVFP4 compressed rows (288 B).
CSA_DECODE_1M_V41 = CSA_DECODE_1M_FP8.with_(name="csa_decode_1m_v41", kv_fmt="mxfp8", comp_fmt="nvfp4")

ALL = [TINY_CSA, CSA_DECODE, HCA_DECODE, CSA_PREFILL, CSA_DECODE_1M_FP8, CSA_DECODE_1M_V41]
BY_NAME = {w.name: w for w in ALL}
