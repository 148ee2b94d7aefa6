"""Python binding of libhcs.so, the C-ABI library of the hybrid compressed sparse attention path.

Argument marshalling only: torch tensors become device pointers and the current HIP stream;
every step of the path runs in the library's HIP kernels. The functions mirror the C entry
points of ``include/hcs.h`` (``hcs_compress_kv`` -> ``compress_kv`` and so on) and return
nothing; a non-OK status raises ``HcsError`` with the library's message.

There is no fallback: if ``libhcs.so`` is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhcs.so")

FMT = {"bf16": 0, "fp8ds": 1, "mxfp4": 2, "fp8ix": 3, "mxfp8": 4, "nvfp4": 5}
IN_DTYPE = {torch.bfloat16: 0, torch.float32: 1}


class HcsError(RuntimeError):
    pass


class Paged(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("page_table", ctypes.c_void_p),
                ("pt_stride", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("fmt", ctypes.c_int32), ("dim", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise HcsError(f"{LIB_PATH} is not built (python -m hybrid_compressed_sparse_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        L.hcs_last_error.restype = ctypes.c_char_p
        L.hcs_abi_version.restype = i32
        L.hcs_device_errors.restype = i32
        L.hcs_device_errors.argtypes = [ctypes.POINTER(ctypes.c_uint32), i32]
        L.hcs_compress_kv.restype = i32
        L.hcs_compress_kv.argtypes = [vp, vp, i32, i64, vp, vp, i32, i32, i32, i32, vp, vp, Paged,
                                      vp, i64, vp]
        L.hcs_compress_kv_full.restype = i32
        L.hcs_compress_kv_full.argtypes = [vp, vp, i32, i64, vp, vp, i32, i32, i32, i32, i32, vp, vp,
                                           vp, ctypes.c_float, vp, vp, i32, i32, Paged, vp, i64, vp]
        L.hcs_index_topk_workspace_size.restype = sz
        L.hcs_index_topk_workspace_size.argtypes = [i32, i32, i32, i32]
        L.hcs_index_topk.restype = i32
        L.hcs_index_topk.argtypes = [vp, vp, vp, Paged, vp, vp, i32, i32, i32, i32, i32, i32, vp, vp,
                                     vp, sz, vp]
        L.hcs_index_topk_chunk.restype = i32
        L.hcs_index_topk_chunk.argtypes = [vp, vp, vp, Paged, i32, i32, i32, i32, i32, i32, i32, vp, vp,
                                           vp, sz, vp]
        L.hcs_index_topk_compress.restype = i32
        L.hcs_index_topk_compress.argtypes = [vp, vp, vp, Paged, vp, vp, i32, i32, i32, i32, i32, i32,
                                              vp, vp, vp, sz, vp, vp, i32, i64, vp, vp, i32, i32, i32,
                                              i32, vp, vp, Paged, vp]
        L.hcs_index_scores_compress.restype = i32
        L.hcs_index_scores_compress.argtypes = [vp, vp, vp, Paged, vp, vp, i32, i32, i32, i32, i32, vp, i64,
                                                vp, vp, i32, i64, vp, vp, i32, i32, i32, i32, vp, vp, Paged,
                                                vp]
        L.hcs_sparse_mla_decode_select.restype = i32
        L.hcs_sparse_mla_decode_select.argtypes = [vp, Paged, Paged, vp, i64, i32, vp, vp, vp, i32, i32,
                                                   i32, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
        L.hcs_sparse_mla_workspace_size.restype = sz
        L.hcs_sparse_mla_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.hcs_sparse_mla_decode.restype = i32
        L.hcs_sparse_mla_decode.argtypes = [vp, Paged, Paged, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                            i32, i32, f32, vp, vp, vp, sz, vp]
        L.hcs_sparse_mla_decode_noalloc.restype = i32
        L.hcs_sparse_mla_decode_noalloc.argtypes = [vp, Paged, Paged, vp, i32, vp, vp, vp, i32, i32, i32, i32,
                                                    i32, i32, f32, vp, vp, vp]
        L.hcs_sparse_mla_prefill_workspace_size.restype = sz
        L.hcs_sparse_mla_prefill_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32]
        L.hcs_sparse_mla_prefill_chunk.restype = i32
        L.hcs_sparse_mla_prefill_chunk.argtypes = [vp, Paged, Paged, vp, i32, i32, i32, i32, vp, i32,
                                                   i32, i32, i32, f32, vp, vp, vp, sz, vp]
        L.hcs_qnorm_rope_kv_insert.restype = i32
        L.hcs_qnorm_rope_kv_insert.argtypes = [vp, i32, vp, i64, vp, vp, i32, i32, i32, ctypes.c_float,
                                               vp, vp, i32, i32, Paged, vp]
        L.hcs_indexer_q_prep.restype = i32
        L.hcs_indexer_q_prep.argtypes = [vp, vp, vp, i32, i32, i32, f32, vp, vp, i32, i32, i32, vp, vp, vp, vp]
        L.hcs_indexer_k_store.restype = i32
        L.hcs_indexer_k_store.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, f32, vp, vp, i32, i32, Paged, vp]
        L.hcs_index_topk_cand_workspace_size.restype = sz
        L.hcs_index_topk_cand_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
        L.hcs_index_topk_cand.restype = i32
        L.hcs_index_topk_cand.argtypes = [vp, vp, vp, Paged, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                          vp, vp, vp, vp, vp, sz, vp]
        _lib = L
    return _lib


DEVERR_PAGE_RANGE = 0x1   # a page-table entry >= num_pages was met
DEVERR_PAIR_WAIT = 0x2    # the prefill attention's head-pair exchange timed out


def device_errors(clear: bool = True) -> int:
    """hcs_device_errors: waits for the current device, returns its error bits (DEVERR_*) and
    clears them unless clear is False."""
    v = ctypes.c_uint32(0)
    _check(lib().hcs_device_errors(ctypes.byref(v), 1 if clear else 0), "device_errors")
    return int(v.value)


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = lib().hcs_last_error().decode()
        raise HcsError(f"{what} failed with status {status}: {msg}")


def _ptr(t: Optional[torch.Tensor], dtype=None, name: str = "tensor"):
    if t is None:
        return None
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def paged(pool: torch.Tensor, page_table: torch.Tensor, fmt: str, dim: int) -> Paged:
    """A paged cache: pool uint8 [num_pages, page_bytes], page_table int32 [num_seqs, pt_stride].
    The descriptor holds references to both tensors, so their memory stays allocated for as long
    as the descriptor lives (it carries only their addresses to the library)."""
    if pool.dtype != torch.uint8 or page_table.dtype != torch.int32:
        raise TypeError("pool must be uint8 and page_table int32")
    p = Paged(_ptr(pool, name="pool"), _ptr(page_table, name="page_table"), page_table.shape[-1],
              pool.shape[0], FMT[fmt], dim)
    p._tensors = (pool, page_table)
    return p


def _as_paged(c) -> Paged:
    return c if isinstance(c, Paged) else paged(c.pool, c.page_table, c.fmt, c.dim)


def _workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """A workspace of nbytes (None when none is needed); the library needs no initial contents."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------ compressor

def compress_kv(kv: torch.Tensor, score: torch.Tensor, cu_new: torch.Tensor, start_pos: torch.Tensor,
                state: torch.Tensor, comp, m: int, ape: Optional[torch.Tensor] = None,
                dbg: Optional[torch.Tensor] = None, max_new: Optional[int] = None) -> None:
    """hcs_compress_kv. kv, score [T, d] (bf16 or f32); cu_new [B+1], start_pos [B] int32;
    state [B, 3d] f32; comp: paged cache (bf16 or fp8ds); dbg [B, rows, d] f32 or None."""
    if kv.dtype != score.dtype or kv.dtype not in IN_DTYPE:
        raise TypeError("kv and score must both be bf16 or both float32")
    B = start_pos.shape[0]
    d = kv.shape[-1]
    if max_new is None:
        raise ValueError("max_new (host bound of new tokens per sequence) is required")
    _check(lib().hcs_compress_kv(
        _ptr(kv, name="kv"), _ptr(score, name="score"), IN_DTYPE[kv.dtype], kv.stride(0),
        _ptr(cu_new, torch.int32, "cu_new"), _ptr(start_pos, torch.int32, "start_pos"), B, max_new, d, m,
        _ptr(ape, torch.float32, "ape"), _ptr(state, torch.float32, "state"), _as_paged(comp),
        _ptr(dbg, torch.float32, "dbg"), 0 if dbg is None else dbg.stride(0), _stream()), "compress_kv")


def compress_kv_full(kv: torch.Tensor, score: torch.Tensor, cu_new: torch.Tensor, start_pos: torch.Tensor,
                     state: torch.Tensor, comp, m: int, coff: int, ape: Optional[torch.Tensor] = None,
                     norm_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
                     rope_cos: Optional[torch.Tensor] = None, rope_sin: Optional[torch.Tensor] = None,
                     dbg: Optional[torch.Tensor] = None, max_new: Optional[int] = None) -> None:
    """hcs_compress_kv_full. kv, score [T, coff*d] (bf16 or f32); state [B, 3*coff*d] f32;
    norm_weight [d] f32; rope_cos / rope_sin [rows, d_rope/2] f32 (d_rope = 2 * columns)."""
    if kv.dtype != score.dtype or kv.dtype not in IN_DTYPE:
        raise TypeError("kv and score must both be bf16 or both float32")
    if max_new is None:
        raise ValueError("max_new (host bound of new tokens per sequence) is required")
    B = start_pos.shape[0]
    d = kv.shape[-1] // coff
    d_rope = 0 if rope_cos is None else 2 * rope_cos.shape[-1]
    rows = 0 if rope_cos is None else rope_cos.shape[0]
    _check(lib().hcs_compress_kv_full(
        _ptr(kv, name="kv"), _ptr(score, name="score"), IN_DTYPE[kv.dtype], kv.stride(0),
        _ptr(cu_new, torch.int32, "cu_new"), _ptr(start_pos, torch.int32, "start_pos"), B, max_new, d, m,
        coff, _ptr(ape, torch.float32, "ape"), _ptr(state, torch.float32, "state"),
        _ptr(norm_weight, torch.float32, "norm_weight"), norm_eps, _ptr(rope_cos, torch.float32, "rope_cos"),
        _ptr(rope_sin, torch.float32, "rope_sin"), d_rope, rows, _as_paged(comp),
        _ptr(dbg, torch.float32, "dbg"), 0 if dbg is None else dbg.stride(0), _stream()), "compress_kv_full")


# ------------------------------------------------------------------------------ query prep + SWA insert

def qnorm_rope_kv_insert(q: Optional[torch.Tensor], kv: Optional[torch.Tensor], tok_seq: Optional[torch.Tensor],
                         tok_pos: torch.Tensor, swa=None, rope_cos: Optional[torch.Tensor] = None,
                         rope_sin: Optional[torch.Tensor] = None, q_norm: bool = False,
                         eps: float = 1e-6, d: Optional[int] = None) -> None:
    """hcs_qnorm_rope_kv_insert. q [N, H, d] bf16 (in place) or None; kv [N, >= d] bf16 rows
    (row stride kv.stride(0)) or None; tok_seq, tok_pos [N] int32; rope_cos / rope_sin
    [rows, d_rope/2] f32 (d_rope = 2 * columns); swa: the sliding-window cache."""
    if q is not None and q.dtype != torch.bfloat16:
        raise TypeError("q must be bf16")
    if kv is not None and (kv.dtype != torch.bfloat16 or kv.stride(1) != 1):
        raise TypeError("kv must be bf16 rows with unit column stride")
    N = tok_pos.shape[0]
    H = 0 if q is None else q.shape[1]
    if d is None:
        d = q.shape[2] if q is not None else swa.dim
    d_rope = 0 if rope_cos is None else 2 * rope_cos.shape[-1]
    rows = 0 if rope_cos is None else rope_cos.shape[0]
    kv_ptr = None
    if kv is not None:
        if not kv.is_cuda:
            raise ValueError("kv must be on the GPU")
        kv_ptr = kv.data_ptr()
    sw = _as_paged(swa) if swa is not None else Paged(None, None, 0, 0, 0, d)
    _check(lib().hcs_qnorm_rope_kv_insert(
        _ptr(q, torch.bfloat16, "q"), H, kv_ptr, 0 if kv is None else kv.stride(0),
        _ptr(tok_seq, torch.int32, "tok_seq"), _ptr(tok_pos, torch.int32, "tok_pos"), N, d,
        1 if q_norm else 0, eps, _ptr(rope_cos, torch.float32, "rope_cos"),
        _ptr(rope_sin, torch.float32, "rope_sin"), d_rope, rows, sw, _stream()), "qnorm_rope_kv_insert")


# ------------------------------------------------------------------------------ indexer Q / K production

def indexer_q_prep(q: torch.Tensor, w: torch.Tensor, tok_pos: torch.Tensor, out_fmt: str, q_out: torch.Tensor,
                   w_out: torch.Tensor, q_scale_out: Optional[torch.Tensor] = None, w_scale: float = 1.0,
                   rope_cos: Optional[torch.Tensor] = None, rope_sin: Optional[torch.Tensor] = None) -> None:
    """hcs_indexer_q_prep. q [N, H_I, 128] bf16, w [N, H_I] f32, tok_pos [N] int32; out_fmt
    "bf16" (q_out bf16 [N, H_I, 128]), "mxfp4" (q_out uint8 [N, H_I, 64], q_scale_out uint8
    [N, H_I, 4]) or "fp8ix" (q_out uint8 [N, H_I, 128], q_scale_out f32 [N, H_I])."""
    N, H, d = q.shape
    d_rope = 0 if rope_cos is None else 2 * rope_cos.shape[-1]
    rows = 0 if rope_cos is None else rope_cos.shape[0]
    _check(lib().hcs_indexer_q_prep(
        _ptr(q, torch.bfloat16, "q"), _ptr(w, torch.float32, "w"), _ptr(tok_pos, torch.int32, "tok_pos"), N, H, d,
        w_scale, _ptr(rope_cos, torch.float32, "rope_cos"), _ptr(rope_sin, torch.float32, "rope_sin"), d_rope, rows,
        FMT[out_fmt], _ptr(q_out, name="q_out"), _ptr(q_scale_out, name="q_scale_out"),
        _ptr(w_out, torch.float32, "w_out"), _stream()), "indexer_q_prep")


def indexer_k_store(k_pre: torch.Tensor, ent_seq: torch.Tensor, ent_idx: torch.Tensor, m: int, keys,
                    norm_weight: torch.Tensor, eps: float = 1e-6, rope_cos: Optional[torch.Tensor] = None,
                    rope_sin: Optional[torch.Tensor] = None) -> None:
    """hcs_indexer_k_store. k_pre [n, >= 128] bf16 rows (row stride k_pre.stride(0)); ent_seq,
    ent_idx [n] int32; keys: the indexer key cache (bf16, mxfp4 or fp8ix, dim 128)."""
    if k_pre.dtype != torch.bfloat16 or k_pre.stride(1) != 1 or not k_pre.is_cuda:
        raise TypeError("k_pre must be bf16 rows on the GPU with unit column stride")
    d_rope = 0 if rope_cos is None else 2 * rope_cos.shape[-1]
    rows = 0 if rope_cos is None else rope_cos.shape[0]
    _check(lib().hcs_indexer_k_store(
        k_pre.data_ptr(), k_pre.stride(0), _ptr(ent_seq, torch.int32, "ent_seq"), _ptr(ent_idx, torch.int32, "ent_idx"),
        ent_idx.shape[0], 128, m, _ptr(norm_weight, torch.float32, "norm_weight"), eps,
        _ptr(rope_cos, torch.float32, "rope_cos"), _ptr(rope_sin, torch.float32, "rope_sin"), d_rope, rows,
        _as_paged(keys), _stream()), "indexer_k_store")


# ------------------------------------------------------------------------------ indexer

def index_topk_workspace_size(N: int, max_pos: int, m: int, topk: int) -> int:
    return lib().hcs_index_topk_workspace_size(N, max_pos, m, topk)


def index_topk(q, q_scale: Optional[torch.Tensor], w: torch.Tensor, keys, q_seq: torch.Tensor,
               q_pos: torch.Tensor, m: int, topk: int, max_pos: int, out_idx: torch.Tensor,
               out_score: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> None:
    """hcs_index_topk. q: bf16 [N, H_I, d_I] (bf16 keys) or uint8 [N, H_I, d_I/2] with
    q_scale uint8 [N, H_I, d_I/32] (mxfp4 keys); w f32 [N, H_I]; out_idx int32 [N, topk]."""
    N, H_I = w.shape
    d_I = keys.dim
    if ws is None:
        ws = _workspace(index_topk_workspace_size(N, max_pos, m, topk), w.device)
    _check(lib().hcs_index_topk(
        _ptr(q, name="q"), _ptr(q_scale, name="q_scale"), _ptr(w, torch.float32, "w"),
        _as_paged(keys), _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"),
        N, H_I, d_I, m, topk, max_pos, _ptr(out_idx, torch.int32, "out_idx"),
        _ptr(out_score, torch.float32, "out_score"), _ptr(ws, name="ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()), "index_topk")


def index_topk_cand(q, q_scale: Optional[torch.Tensor], w: torch.Tensor, keys, q_seq: torch.Tensor,
                    q_pos: torch.Tensor, m: int, topk: int, max_pos: int, cand_block: int, n_cand: int,
                    out_idx: torch.Tensor, cand_in: Optional[torch.Tensor] = None,
                    cand_out: Optional[torch.Tensor] = None, out_score: Optional[torch.Tensor] = None,
                    ws: Optional[torch.Tensor] = None) -> None:
    """hcs_index_topk_cand: index_topk plus two-level candidate filtering; give cand_out
    (int32 [N, n_cand], source) or cand_in (int32 [N, n_cand], consumer)."""
    N, H_I = w.shape
    d_I = keys.dim
    if ws is None:
        n = lib().hcs_index_topk_cand_workspace_size(N, max_pos, m, topk, cand_block, n_cand)
        ws = _workspace(n, w.device)
    _check(lib().hcs_index_topk_cand(
        _ptr(q, name="q"), _ptr(q_scale, name="q_scale"), _ptr(w, torch.float32, "w"), _as_paged(keys),
        _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"), N, H_I, d_I, m, topk, max_pos,
        cand_block, n_cand, _ptr(cand_in, torch.int32, "cand_in"), _ptr(cand_out, torch.int32, "cand_out"),
        _ptr(out_idx, torch.int32, "out_idx"), _ptr(out_score, torch.float32, "out_score"), _ptr(ws, name="ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()), "index_topk_cand")


def index_topk_chunk(q, q_scale: Optional[torch.Tensor], w: torch.Tensor, keys, seq: int, P0: int,
                     m: int, topk: int, out_idx: torch.Tensor, out_score: Optional[torch.Tensor] = None,
                     ws: Optional[torch.Tensor] = None) -> None:
    """hcs_index_topk_chunk: index_topk for the queries P0 .. P0+Q-1 of sequence `seq`
    (Q = w.shape[0])."""
    Q, H_I = w.shape
    d_I = keys.dim
    if ws is None:
        ws = _workspace(index_topk_workspace_size(Q, P0 + Q - 1, m, topk), w.device)
    _check(lib().hcs_index_topk_chunk(
        _ptr(q, name="q"), _ptr(q_scale, name="q_scale"), _ptr(w, torch.float32, "w"),
        _as_paged(keys), seq, P0, Q, H_I, d_I, m, topk, _ptr(out_idx, torch.int32, "out_idx"),
        _ptr(out_score, torch.float32, "out_score"), _ptr(ws, name="ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()), "index_topk_chunk")


def index_topk_compress(q, q_scale: Optional[torch.Tensor], w: torch.Tensor, keys, q_seq: torch.Tensor,
                        q_pos: torch.Tensor, m_ix: int, topk: int, max_pos: int, out_idx: torch.Tensor,
                        out_score: Optional[torch.Tensor], ws: Optional[torch.Tensor],
                        kv: torch.Tensor, score: torch.Tensor, cu_new: torch.Tensor,
                        start_pos: torch.Tensor, state: torch.Tensor, comp, m: int,
                        ape: Optional[torch.Tensor] = None, max_new: Optional[int] = None) -> None:
    """hcs_index_topk_compress: index_topk(q .. ws) and compress_kv(kv .. m, ape) of one decode
    step in one launch."""
    N, H_I = w.shape
    d_I = keys.dim
    if kv.dtype != score.dtype or kv.dtype not in IN_DTYPE:
        raise TypeError("kv and score must both be bf16 or both float32")
    if max_new is None:
        raise ValueError("max_new (host bound of new tokens per sequence) is required")
    if ws is None:
        ws = _workspace(index_topk_workspace_size(N, max_pos, m_ix, topk), w.device)
    _check(lib().hcs_index_topk_compress(
        _ptr(q, name="q"), _ptr(q_scale, name="q_scale"), _ptr(w, torch.float32, "w"),
        _as_paged(keys), _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"),
        N, H_I, d_I, m_ix, topk, max_pos, _ptr(out_idx, torch.int32, "out_idx"),
        _ptr(out_score, torch.float32, "out_score"), _ptr(ws, name="ws"),
        0 if ws is None else ws.numel() * ws.element_size(),
        _ptr(kv, name="kv"), _ptr(score, name="score"), IN_DTYPE[kv.dtype], kv.stride(0),
        _ptr(cu_new, torch.int32, "cu_new"), _ptr(start_pos, torch.int32, "start_pos"),
        start_pos.shape[0], max_new, kv.shape[-1], m, _ptr(ape, torch.float32, "ape"),
        _ptr(state, torch.float32, "state"), _as_paged(comp), _stream()), "index_topk_compress")


def index_scores_compress(q, q_scale: Optional[torch.Tensor], w: torch.Tensor, keys, q_seq: torch.Tensor,
                          q_pos: torch.Tensor, m_ix: int, max_pos: int, scores: torch.Tensor,
                          kv: Optional[torch.Tensor] = None, score: Optional[torch.Tensor] = None,
                          cu_new: Optional[torch.Tensor] = None, start_pos: Optional[torch.Tensor] = None,
                          state: Optional[torch.Tensor] = None, comp=None, m: int = 1,
                          ape: Optional[torch.Tensor] = None, max_new: Optional[int] = None) -> None:
    """hcs_index_scores_compress: the indexer scores float32 [N, >= n_visible] (no top-k) and,
    when kv is given, compress_kv(kv .. m, ape) of the same decode step in the same launch."""
    N, H_I = w.shape
    d_I = keys.dim
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise TypeError("scores must be float32 [N, stride] with unit column stride")
    B = 0
    in_dtype, row_stride, d = 0, 0, 0
    if kv is not None:
        if kv.dtype != score.dtype or kv.dtype not in IN_DTYPE:
            raise TypeError("kv and score must both be bf16 or both float32")
        if max_new is None:
            raise ValueError("max_new (host bound of new tokens per sequence) is required")
        B, in_dtype, row_stride, d = start_pos.shape[0], IN_DTYPE[kv.dtype], kv.stride(0), kv.shape[-1]
    _check(lib().hcs_index_scores_compress(
        _ptr(q, name="q"), _ptr(q_scale, name="q_scale"), _ptr(w, torch.float32, "w"),
        _as_paged(keys), _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"),
        N, H_I, d_I, m_ix, max_pos, scores.data_ptr(), scores.stride(0),
        _ptr(kv, name="kv"), _ptr(score, name="score"), in_dtype, row_stride,
        _ptr(cu_new, torch.int32, "cu_new"), _ptr(start_pos, torch.int32, "start_pos"),
        B, max_new or 0, d, m, _ptr(ape, torch.float32, "ape"), _ptr(state, torch.float32, "state"),
        _as_paged(comp) if comp is not None else Paged(), _stream()), "index_scores_compress")


# ------------------------------------------------------------------------------ attention

def sparse_mla_workspace_size(N: int, H: int, d: int, window: int, m: int, topk: int, max_pos: int) -> int:
    return lib().hcs_sparse_mla_workspace_size(N, H, d, window, m, topk, max_pos)


def sparse_mla_decode(q: torch.Tensor, swa, comp, topk_idx: Optional[torch.Tensor], q_seq: torch.Tensor,
                      q_pos: torch.Tensor, window: int, m: int, max_pos: int, scale: float,
                      out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                      sink: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> None:
    """hcs_sparse_mla_decode. q, out bf16 [N, H, d]; topk_idx int32 [N, k] or None (HCA)."""
    N, H, d = q.shape
    topk = 0 if topk_idx is None else topk_idx.shape[1]
    if ws is None:
        ws = _workspace(sparse_mla_workspace_size(N, H, d, window, m, topk, max_pos), q.device)
    _check(lib().hcs_sparse_mla_decode(
        _ptr(q, torch.bfloat16, "q"), _as_paged(swa), _as_paged(comp), _ptr(topk_idx, torch.int32, "topk_idx"),
        topk, _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"),
        _ptr(sink, torch.float32, "sink"), N, H, d, window, m, max_pos, scale,
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _ptr(ws, name="ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()), "sparse_mla_decode")


def sparse_mla_decode_noalloc(q: torch.Tensor, swa, comp, topk_idx: Optional[torch.Tensor], q_seq: torch.Tensor,
                              q_pos: torch.Tensor, window: int, m: int, max_pos: int, scale: float,
                              out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                              sink: Optional[torch.Tensor] = None) -> None:
    """hcs_sparse_mla_decode_noalloc: hcs_sparse_mla_decode with the library's static scratch
    instead of a workspace (nothing is allocated)."""
    N, H, d = q.shape
    topk = 0 if topk_idx is None else topk_idx.shape[1]
    _check(lib().hcs_sparse_mla_decode_noalloc(
        _ptr(q, torch.bfloat16, "q"), _as_paged(swa), _as_paged(comp), _ptr(topk_idx, torch.int32, "topk_idx"),
        topk, _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"),
        _ptr(sink, torch.float32, "sink"), N, H, d, window, m, max_pos, scale,
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _stream()), "sparse_mla_decode_noalloc")


def sparse_mla_decode_select(q: torch.Tensor, swa, comp, scores: torch.Tensor, topk: int,
                             q_seq: torch.Tensor, q_pos: torch.Tensor, window: int, m: int, max_pos: int,
                             scale: float, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                             sel_idx: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None,
                             ws: Optional[torch.Tensor] = None) -> None:
    """hcs_sparse_mla_decode_select: CSA decode attention that takes each query's top-k of the
    indexer scores (float32 [N, >= n_visible]) itself; sel_idx int32 [N, topk] receives the
    selected ids in ascending order (-1 padded) when given."""
    N, H, d = q.shape
    if scores.dtype != torch.float32 or scores.dim() != 2 or scores.stride(1) != 1:
        raise TypeError("scores must be float32 [N, stride] with unit column stride")
    if ws is None:
        ws = _workspace(sparse_mla_workspace_size(N, H, d, window, m, topk, max_pos), q.device)
    _check(lib().hcs_sparse_mla_decode_select(
        _ptr(q, torch.bfloat16, "q"), _as_paged(swa), _as_paged(comp), scores.data_ptr(), scores.stride(0),
        topk, _ptr(q_seq, torch.int32, "q_seq"), _ptr(q_pos, torch.int32, "q_pos"),
        _ptr(sink, torch.float32, "sink"), N, H, d, window, m, max_pos, scale,
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"),
        _ptr(sel_idx, torch.int32, "sel_idx"), _ptr(ws, name="ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()), "sparse_mla_decode_select")


def sparse_mla_prefill_workspace_size(Q: int, H: int, d: int, window: int, m: int, topk: int, P0: int) -> int:
    return lib().hcs_sparse_mla_prefill_workspace_size(Q, H, d, window, m, topk, P0)


def sparse_mla_prefill_chunk(q: torch.Tensor, swa, comp, topk_idx: Optional[torch.Tensor], seq: int,
                             P0: int, window: int, m: int, scale: float, out: torch.Tensor,
                             lse: Optional[torch.Tensor] = None, sink: Optional[torch.Tensor] = None,
                             ws: Optional[torch.Tensor] = None) -> None:
    """hcs_sparse_mla_prefill_chunk for queries P0 .. P0+Q-1 of sequence `seq`."""
    Q, H, d = q.shape
    topk = 0 if topk_idx is None else topk_idx.shape[1]
    if ws is None:
        ws = _workspace(sparse_mla_prefill_workspace_size(Q, H, d, window, m, topk, P0), q.device)
    _check(lib().hcs_sparse_mla_prefill_chunk(
        _ptr(q, torch.bfloat16, "q"), _as_paged(swa), _as_paged(comp), _ptr(topk_idx, torch.int32, "topk_idx"),
        topk, seq, P0, Q, _ptr(sink, torch.float32, "sink"), H, d, window, m, scale,
        _ptr(out, torch.bfloat16, "out"), _ptr(lse, torch.float32, "lse"), _ptr(ws, name="ws"),
        0 if ws is None else ws.numel() * ws.element_size(), _stream()), "sparse_mla_prefill_chunk")
