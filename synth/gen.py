"""Seeded generators for the workloads in ``synth.configs``.

Every tensor is drawn from its own ``torch.Generator`` seeded from (seed, tag),
so a tensor does not depend on which others were drawn first. Draws happen on
the requested device; CPU and GPU draws of the same seed differ, and every
consumer (GPU path, oracle) reads the same drawn tensors, never a redraw.

Stored formats are produced here only to *make inputs*: bf16 by torch's
round-to-nearest-even cast, fp8_ds by torch's float8_e4m3fn cast after a
power-of-two block scale, MXFP4 by nearest e2m1 magnitude after a power-of-two
block scale. The path under test never calls these.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field
from typing import Optional

import torch

from . import layout as L
from .configs import Workload

def _gen(seed: int, tag: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 0x9E3779B1 + zlib.crc32(tag.encode())) % (2 ** 62))
    return g


def randn(seed, tag, shape, device, std=1.0) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(seed, tag, device), device=device,
                       dtype=torch.float32) * std


def rand(seed, tag, shape, device) -> torch.Tensor:
    return torch.rand(shape, generator=_gen(seed, tag, device), device=device, dtype=torch.float32)


def randperm(seed, tag, n, device) -> torch.Tensor:
    return torch.randperm(n, generator=_gen(seed, tag, device), device=device)


# ---------------------------------------------------------------- input encoders

def _pow2_exponent_for(amax: torch.Tensor, qmax: float) -> torch.Tensor:
    """Smallest integer e with amax / 2**e <= qmax (e = 0 where amax == 0), clamped to [-127, 127]."""
    mant, expo = torch.frexp(amax / qmax)
    e = torch.where(mant == 0.5, expo - 1, expo)
    e = torch.where(amax == 0, torch.zeros_like(e), e)
    return e.clamp(-127, 127)


def make_fp8ds(x: torch.Tensor) -> L.Fp8dsRows:
    """fp8_ds rows from float values [..., 512]."""
    lead = x.shape[:-1]
    lat = x[..., :L.FP8DS_LATENT].float().reshape(*lead, L.FP8DS_NSCALE, L.FP8DS_BLOCK)
    e = _pow2_exponent_for(lat.abs().amax(-1), 448.0)
    y = lat * torch.pow(2.0, -e.float())[..., None]
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, L.FP8DS_LATENT)
    return L.Fp8dsRows(codes=codes, rope=x[..., L.FP8DS_LATENT:].to(torch.bfloat16),
                       scales=(e + 127).to(torch.uint8))


_E2M1_MAG = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def make_mxfp4(x: torch.Tensor) -> L.Mxfp4Rows:
    """MXFP4 rows from float values [..., D]: element 2j in the low nibble of byte j."""
    lead, D = x.shape[:-1], x.shape[-1]
    blk = x.float().reshape(*lead, D // L.MX_BLOCK, L.MX_BLOCK)
    e = _pow2_exponent_for(blk.abs().amax(-1), 6.0)
    y = blk * torch.pow(2.0, -e.float())[..., None]
    mags = _E2M1_MAG.to(x.device)
    code = (y.abs()[..., None] - mags).abs().argmin(-1).to(torch.uint8)
    code = code | ((y < 0).to(torch.uint8) << 3)
    code = code.reshape(*lead, D)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return L.Mxfp4Rows(codes=packed.contiguous(), scales=(e + 127).to(torch.uint8))


def make_mxfp8(x: torch.Tensor) -> L.Mxfp4Rows:
    """MXFP8 rows (512 e4m3 + one power-of-two scale per 32) from float values [..., 512]."""
    lead = x.shape[:-1]
    blk = x.float().reshape(*lead, L.V41_DIM // L.MXFP8_BLOCK, L.MXFP8_BLOCK)
    e = _pow2_exponent_for(blk.abs().amax(-1), 448.0)
    y = blk * torch.pow(2.0, -e.float())[..., None]
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).reshape(*lead, L.V41_DIM)
    return L.Mxfp4Rows(codes=codes, scales=(e + 127).to(torch.uint8))


def make_nvfp4(x: torch.Tensor) -> L.Mxfp4Rows:
    """NVFP4 rows (512 e2m1, element 2j in the low nibble, + one e4m3 scale per 16) from float
    values [..., 512]: the scale is torch's e4m3 cast of amax / 6, the codes the nearest e2m1
    magnitude of x / scale (clamped to 6)."""
    lead = x.shape[:-1]
    blk = x.float().reshape(*lead, L.V41_DIM // L.NVFP4_BLOCK, L.NVFP4_BLOCK)
    s8 = (blk.abs().amax(-1) / 6.0).clamp(max=448.0).to(torch.float8_e4m3fn)
    sv = s8.float()
    y = torch.where(sv[..., None] > 0, blk / sv.clamp(min=1e-30)[..., None], torch.zeros_like(blk)).clamp(-6, 6)
    mags = _E2M1_MAG.to(x.device)
    code = (y.abs()[..., None] - mags).abs().argmin(-1).to(torch.uint8)
    code = (code | ((y < 0).to(torch.uint8) << 3)).reshape(*lead, L.V41_DIM)
    packed = code[..., 0::2] | (code[..., 1::2] << 4)
    return L.Mxfp4Rows(codes=packed.contiguous(), scales=s8.view(torch.uint8))


def encode_rows(x: torch.Tensor, fmt: str):
    if fmt == L.FMT_BF16:
        return x.to(torch.bfloat16)
    if fmt == L.FMT_FP8DS:
        return make_fp8ds(x)
    if fmt == L.FMT_MXFP4:
        return make_mxfp4(x)
    if fmt == L.FMT_MXFP8:
        return make_mxfp8(x)
    if fmt == L.FMT_NVFP4:
        return make_nvfp4(x)
    raise ValueError(fmt)


def rows_index(rows, idx):
    return rows[idx] if isinstance(rows, torch.Tensor) else rows.index(idx)


def rows_to(rows, device):
    return rows.to(device)


# ---------------------------------------------------------------- paged caches

@dataclass
class PagedCache:
    """A paged cache pool plus the logical rows it holds (codes, per sequence)."""
    fmt: str
    dim: int
    pool: torch.Tensor            # uint8 [num_pages, page_bytes]
    page_table: torch.Tensor      # int32 [B, pt_width], -1 = not resident
    lo: list                      # per sequence: first logical row held
    rows: list                    # per sequence: logical rows lo .. lo+len-1 (codes)

    def logical(self, b: int, ids: torch.Tensor):
        """Codes of logical rows ``ids`` of sequence b (from the generated copy)."""
        return rows_index(self.rows[b], ids.long().to(self._dev(b)) - self.lo[b])

    def _dev(self, b):
        r = self.rows[b]
        return r.device if isinstance(r, torch.Tensor) else r.codes.device


def build_paged(seed: int, tag: str, fmt: str, dim: int, spans: list, pt_width: int, device,
                std: float, chunk_rows: int = 1 << 16) -> PagedCache:
    """Random rows ~ N(0, std^2) for logical rows [lo, hi) of each sequence, in random pages."""
    pages_per_seq = []
    for lo, hi in spans:
        first, last = lo // L.PAGE_ROWS, (hi - 1) // L.PAGE_ROWS
        pages_per_seq.append(list(range(first, last + 1)) if hi > lo else [])
    total = sum(len(p) for p in pages_per_seq)
    perm = randperm(seed, tag + ".perm", max(total, 1), device).to(torch.int32)
    pt = torch.full((len(spans), pt_width), -1, dtype=torch.int32, device=device)
    k = 0
    for b, pages in enumerate(pages_per_seq):
        if pages:
            pt[b, pages[0]: pages[-1] + 1] = perm[k: k + len(pages)]
            k += len(pages)
    pool = L.new_pool(max(total, 1), fmt, dim, device)
    rows_all = []
    for b, (lo, hi) in enumerate(spans):
        parts = []
        for c0 in range(lo, hi, chunk_rows):
            c1 = min(hi, c0 + chunk_rows)
            x = randn(seed, f"{tag}.rows.{b}.{c0}", (c1 - c0, dim), device, std)
            enc = encode_rows(x, fmt)
            L.scatter_rows(pool, fmt, dim, pt[b], torch.arange(c0, c1, device=device), enc)
            parts.append(enc)
        rows_all.append(_cat_rows(parts, fmt, dim, device))
    return PagedCache(fmt, dim, pool, pt, [s[0] for s in spans], rows_all)


def _cat_rows(parts, fmt, dim, device):
    if fmt == L.FMT_BF16:
        return torch.cat(parts) if parts else torch.zeros((0, dim), dtype=torch.bfloat16, device=device)
    if not parts:
        parts = [encode_rows(torch.zeros((0, dim), device=device), fmt)]
    if fmt == L.FMT_FP8DS:
        return L.Fp8dsRows(torch.cat([p.codes for p in parts]), torch.cat([p.rope for p in parts]),
                           torch.cat([p.scales for p in parts]))
    return L.Mxfp4Rows(torch.cat([p.codes for p in parts]), torch.cat([p.scales for p in parts]))


# ---------------------------------------------------------------- scenarios

@dataclass
class Scenario:
    """All inputs of one step of the path, on one device."""
    wl: Workload
    seed: int
    device: torch.device
    q_seq: torch.Tensor          # int32 [N]
    q_pos: torch.Tensor          # int32 [N]
    q: torch.Tensor              # bf16 [N, H, d]
    swa: PagedCache              # raw rows by absolute position
    comp: PagedCache             # compressed entries by index
    ix_q: Optional[object]       # bf16 [N, H_I, d_I] or Mxfp4Rows [N, H_I, ...]
    ix_w: Optional[torch.Tensor] # fp32 [N, H_I]
    ix: Optional[PagedCache]     # indexer keys by entry index
    c_start: torch.Tensor        # int32 [B]: position of the first token of each compressor stream
    c_cu: list                   # [B+1] row offsets of each sequence's stream in c_x / c_s
    c_x: torch.Tensor            # [sum T_b, d] raw KV of the compressor streams (in_dtype)
    c_s: torch.Tensor            # [sum T_b, d] gate logits of the compressor streams (in_dtype)
    n_step: int                  # the last n_step tokens of each stream belong to the step itself
    ape: Optional[torch.Tensor] = None   # fp32 [m, d] or None
    extra: dict = field(default_factory=dict)

    @property
    def N(self):
        return self.q_seq.shape[0]

    def max_pos(self) -> int:
        return int(self.q_pos.max().item()) if self.N else 0


def _in_cast(x: torch.Tensor, in_dtype: str) -> torch.Tensor:
    return x.to(torch.bfloat16) if in_dtype == "bf16" else x.float()


def build(wl: Workload, seed: int = 0, device="cpu", ctx_per_seq: Optional[list] = None,
          q_gain: float = 1.0, ape: bool = False, with_swa_from_stream: Optional[bool] = None,
          stream_tokens: Optional[int] = None) -> Scenario:
    """Build one step's inputs for workload ``wl``.

    ctx_per_seq: decode only, per-sequence context length (ragged batches).
    q_gain: multiplies q (sharper attention logits).
    ape: draw an absolute positional encoding [m, d] for the compressor gate logits.
    stream_tokens: decode only, tokens of the compressor stream (default m: the block ending at the query).
    """
    device = torch.device(device)
    d, m, w = wl.d, wl.m, wl.window
    q_std = (wl.q_std or 1.0 / math.sqrt(d)) * q_gain
    kv_std = 1.0 / math.sqrt(d)

    if wl.kind == "decode":
        ctx = list(ctx_per_seq) if ctx_per_seq is not None else [wl.ctx] * wl.B
        B = len(ctx)
        q_seq = torch.arange(B, dtype=torch.int32)
        q_pos = torch.tensor([c - 1 for c in ctx], dtype=torch.int32)
        T = stream_tokens if stream_tokens is not None else m
        c_start = [max(0, ((c - 1) // m) * m - (T - m)) for c in ctx]
        c_len = [c - s for c, s in zip(ctx, c_start)]
        n_step = 1
    elif wl.kind == "tiny":
        B = 1
        ctx = [wl.ctx]
        q_seq = torch.zeros(wl.n_query, dtype=torch.int32)
        q_pos = torch.arange(wl.ctx - wl.n_query, wl.ctx, dtype=torch.int32)
        c_start, c_len = [0], [wl.ctx]
        n_step = wl.ctx
    elif wl.kind == "prefill":
        B = 1
        ctx = [wl.P0 + wl.Q]
        q_seq = torch.zeros(wl.Q, dtype=torch.int32)
        q_pos = torch.arange(wl.P0, wl.P0 + wl.Q, dtype=torch.int32)
        # the stream starts at the block holding P0: tokens before P0 are the previous chunk's
        c0 = (wl.P0 // m) * m
        c_start, c_len = [c0], [wl.P0 + wl.Q - c0]
        n_step = wl.Q
    else:
        raise ValueError(wl.kind)
    N = q_seq.shape[0]
    c_cu = [0]
    for n in c_len:
        c_cu.append(c_cu[-1] + n)

    # queries
    q = (randn(seed, "q", (N, wl.H, d), device, q_std)).to(torch.bfloat16)

    # compressor stream: tokens [c_start, c_start + T) of each sequence
    c_x = randn(seed, "cx", (c_cu[-1], d), device, kv_std)
    c_s = randn(seed, "cs", (c_cu[-1], d), device, 1.0)
    c_x, c_s = _in_cast(c_x, wl.in_dtype), _in_cast(c_s, wl.in_dtype)
    ape_t = randn(seed, "ape", (m, d), device, 1.0) if ape else None

    # sliding-window rows: positions [min_pos - w + 1, max_pos] of each sequence
    pos_host = q_pos.tolist()
    seq_host = q_seq.tolist()
    spans = []
    for b in range(B):
        ps = [p for p, s in zip(pos_host, seq_host) if s == b]
        lo = max(0, min(ps) - w + 1) if ps else 0
        hi = max(ps) + 1 if ps else 0
        spans.append((lo, hi))
    pt_w = (max(ctx) + L.PAGE_ROWS - 1) // L.PAGE_ROWS
    swa = build_paged(seed, "swa", wl.kv_fmt, d, spans, pt_w, device, kv_std)
    from_stream = (wl.kind == "tiny") if with_swa_from_stream is None else with_swa_from_stream
    if from_stream:
        # the sliding-window rows are the compressor's raw KV rows themselves
        for b in range(B):
            lo, hi = spans[b]
            ids = torch.arange(lo, hi, device=device)
            o = c_cu[b] - c_start[b]
            vals = c_x[o + lo: o + hi].float()
            enc = encode_rows(vals, wl.kv_fmt)
            L.scatter_rows(swa.pool, wl.kv_fmt, d, swa.page_table[b], ids, enc)
            swa.rows[b] = enc

    # compressed entries 0 .. n_vis(max pos)-1 (entries the stream completes are rewritten by it)
    n_ent = [(c // m) for c in ctx]
    cpt_w = (max(n_ent) + L.PAGE_ROWS - 1) // L.PAGE_ROWS if max(n_ent) else 1
    comp = build_paged(seed, "comp", wl.cfmt, d, [(0, n) for n in n_ent], cpt_w, device, kv_std)

    ix_q = ix_w = ix = None
    if wl.indexer:
        iq_std = (wl.q_std or 1.0 / math.sqrt(wl.d_I))
        ixq = randn(seed, "ixq", (N, wl.H_I, wl.d_I), device, iq_std)
        ix_q = encode_rows(ixq, wl.ix_fmt)
        ix_w = rand(seed, "ixw", (N, wl.H_I), device)
        ix = build_paged(seed, "ixk", wl.ix_fmt, wl.d_I, [(0, n) for n in n_ent], cpt_w, device,
                         iq_std)

    return Scenario(wl=wl, seed=seed, device=device, q_seq=q_seq.to(device), q_pos=q_pos.to(device),
                    q=q, swa=swa, comp=comp, ix_q=ix_q, ix_w=ix_w, ix=ix,
                    c_start=torch.tensor(c_start, dtype=torch.int32, device=device), c_cu=c_cu,
                    c_x=c_x, c_s=c_s, n_step=n_step, ape=ape_t)
