"""Paged cache byte layouts.

Every cache (sliding-window rows, compressed entries, indexer keys) is a pool of
64-row pages. Logical row r of sequence s lives in page
``page_table[s, r // 64]`` at slot ``r % 64``; a page-table entry of -1 means
the page is not resident.

A page is split into regions, each holding one field of all 64 rows back to
back (structure of arrays inside the page), so every field of every row starts
on an aligned boundary:

  bf16   (dim D)      : [64 x D bf16]
  fp8ds  (dim 512)    : [64 x 448 e4m3 codes][64 x 64 bf16 rope][64 x 8 B: 7 UE8M0 + 1 pad]
                        = 37376 B per page = 584 B per row
  mxfp4  (dim D)      : [64 x D/2 packed e2m1, element 2j in the low nibble][64 x D/32 UE8M0]
                        = 68 B per row for D = 128
  fp8ix  (dim 128)    : [64 x 128 e4m3 codes][64 x float32 scale] = 132 B per row
  mxfp8  (dim 512)    : [64 x 512 e4m3 codes][64 x 16 UE8M0] = 528 B per row
  nvfp4  (dim 512)    : [64 x 256 packed e2m1][64 x 32 e4m3 scales] = 288 B per row

The record widths follow the DeepSeek-V4 pages: 584 B per fp8_ds_mla token
(448 fp8 latent dims + 64 bf16 rotary dims + block scales; "DeepSeek V4.1
attention" API page, KV-cache record section) and 68 B per MXFP4 indexer key
row of 128 dims (same page, indexer K cache row width). The order of the fields
inside a record is not given there; the page-major order above is this
project's choice.

Only byte movement lives here, no arithmetic of the method.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

PAGE_ROWS = 64

FMT_BF16 = "bf16"
FMT_FP8DS = "fp8ds"
FMT_MXFP4 = "mxfp4"
FMT_FP8IX = "fp8ix"
FMT_MXFP8 = "mxfp8"
FMT_NVFP4 = "nvfp4"

FP8DS_DIM = 512
FP8DS_LATENT = 448
FP8DS_ROPE = 64
FP8DS_BLOCK = 64
FP8DS_NSCALE = FP8DS_LATENT // FP8DS_BLOCK  # 7
FP8DS_SCALE_BYTES = 8                       # 7 scales + 1 pad byte
MX_BLOCK = 32
FP8IX_DIM = 128
V41_DIM = 512            # MXFP8 and NVFP4 records hold 512 dims
MXFP8_BLOCK = 32
NVFP4_BLOCK = 16


@dataclass
class Fp8dsRows:
    """Logical fp8_ds rows: e4m3 codes of the latent dims, bf16 rope dims, UE8M0 scales."""
    codes: torch.Tensor   # uint8 [..., 448]
    rope: torch.Tensor    # bfloat16 [..., 64]
    scales: torch.Tensor  # uint8 [..., 7]

    def index(self, idx):
        return Fp8dsRows(self.codes[idx], self.rope[idx], self.scales[idx])

    def to(self, device):
        return Fp8dsRows(self.codes.to(device), self.rope.to(device), self.scales.to(device))


@dataclass
class Mxfp4Rows:
    """Logical MXFP4 rows: packed e2m1 codes (two per byte) and one UE8M0 scale per 32 values."""
    codes: torch.Tensor   # uint8 [..., D/2]
    scales: torch.Tensor  # uint8 [..., D/32]

    def index(self, idx):
        return Mxfp4Rows(self.codes[idx], self.scales[idx])

    def to(self, device):
        return Mxfp4Rows(self.codes.to(device), self.scales.to(device))


@dataclass
class Fp8ixRows:
    """Logical FP8 indexer key rows: 128 e4m3 codes and one float32 scale."""
    codes: torch.Tensor   # uint8 [..., 128]
    scale: torch.Tensor   # float32 [...]

    def index(self, idx):
        return Fp8ixRows(self.codes[idx], self.scale[idx])

    def to(self, device):
        return Fp8ixRows(self.codes.to(device), self.scale.to(device))


def _regions(fmt: str, dim: int):
    """(name, bytes per row) for each region of a page, in page order."""
    if fmt == FMT_BF16:
        return [("row", dim * 2)]
    if fmt == FMT_FP8DS:
        if dim != FP8DS_DIM:
            raise ValueError("fp8ds rows have 512 dims")
        return [("codes", FP8DS_LATENT), ("rope", FP8DS_ROPE * 2), ("scales", FP8DS_SCALE_BYTES)]
    if fmt == FMT_MXFP4:
        if dim % MX_BLOCK:
            raise ValueError("mxfp4 rows need dim % 32 == 0")
        return [("codes", dim // 2), ("scales", dim // MX_BLOCK)]
    if fmt == FMT_FP8IX:
        if dim != FP8IX_DIM:
            raise ValueError("fp8ix rows have 128 dims")
        return [("codes", FP8IX_DIM), ("scale", 4)]
    if fmt in (FMT_MXFP8, FMT_NVFP4):
        if dim != V41_DIM:
            raise ValueError(f"{fmt} rows have 512 dims")
        if fmt == FMT_MXFP8:
            return [("codes", V41_DIM), ("scales", V41_DIM // MXFP8_BLOCK)]
        return [("codes", V41_DIM // 2), ("scales", V41_DIM // NVFP4_BLOCK)]
    raise ValueError(f"unknown format {fmt}")


def row_bytes(fmt: str, dim: int) -> int:
    return sum(b for _, b in _regions(fmt, dim))


def page_bytes(fmt: str, dim: int) -> int:
    return PAGE_ROWS * row_bytes(fmt, dim)


def _row_fields(fmt: str, rows):
    """Byte views [R, bytes] of each region's field for logical rows."""
    if fmt == FMT_BF16:
        r = rows.contiguous()
        return [r.view(torch.uint8).reshape(r.shape[0], -1)]
    if fmt == FMT_FP8DS:
        n = rows.codes.shape[0]
        pad = torch.zeros((n, FP8DS_SCALE_BYTES - FP8DS_NSCALE), dtype=torch.uint8, device=rows.codes.device)
        return [rows.codes.contiguous(),
                rows.rope.contiguous().view(torch.uint8).reshape(n, -1),
                torch.cat([rows.scales, pad], dim=1)]
    if fmt in (FMT_MXFP4, FMT_MXFP8, FMT_NVFP4):
        return [rows.codes.contiguous(), rows.scales.contiguous()]
    if fmt == FMT_FP8IX:
        n = rows.codes.shape[0]
        return [rows.codes.contiguous(), rows.scale.contiguous().view(torch.uint8).reshape(n, 4)]
    raise ValueError(fmt)


def _region_views(buf: torch.Tensor, fmt: str, dim: int):
    """Views [num_pages, 64, bytes] of each region of a page pool."""
    views, off = [], 0
    for _, nb in _regions(fmt, dim):
        views.append(buf[:, off: off + PAGE_ROWS * nb].view(buf.shape[0], PAGE_ROWS, nb))
        off += PAGE_ROWS * nb
    return views


def new_pool(num_pages: int, fmt: str, dim: int, device) -> torch.Tensor:
    return torch.zeros((num_pages, page_bytes(fmt, dim)), dtype=torch.uint8, device=device)


def scatter_rows(buf: torch.Tensor, fmt: str, dim: int, page_table_row: torch.Tensor,
                 logical_ids: torch.Tensor, rows) -> None:
    """Write logical rows ``logical_ids`` of one sequence into the page pool."""
    ids = logical_ids.to(buf.device).long()
    pages = page_table_row.to(buf.device).long()[ids // PAGE_ROWS]
    if bool((pages < 0).any()):
        raise ValueError("row maps to a non-resident page")
    slots = ids % PAGE_ROWS
    for view, field in zip(_region_views(buf, fmt, dim), _row_fields(fmt, rows)):
        view[pages, slots] = field.to(buf.device)


def gather_rows(buf: torch.Tensor, fmt: str, dim: int, page_table_row: torch.Tensor,
                logical_ids: torch.Tensor):
    """Read logical rows ``logical_ids`` of one sequence from the page pool (codes, not values)."""
    ids = logical_ids.to(buf.device).long()
    pages = page_table_row.to(buf.device).long()[ids // PAGE_ROWS]
    slots = ids % PAGE_ROWS
    fields = [v[pages, slots] for v in _region_views(buf, fmt, dim)]
    n = ids.shape[0]
    if fmt == FMT_BF16:
        return fields[0].contiguous().view(torch.bfloat16).reshape(n, dim)
    if fmt == FMT_FP8DS:
        return Fp8dsRows(fields[0].contiguous(), fields[1].contiguous().view(torch.bfloat16).reshape(n, FP8DS_ROPE),
                         fields[2][:, :FP8DS_NSCALE].contiguous())
    if fmt == FMT_FP8IX:
        return Fp8ixRows(fields[0].contiguous(), fields[1].contiguous().view(torch.float32).reshape(n))
    return Mxfp4Rows(fields[0].contiguous(), fields[1].contiguous())
